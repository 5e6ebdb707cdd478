"""Drives the GPU cache (through the C ABI) and the CPU oracle in lockstep and compares them.

The oracle sees the same fp16 inputs, restricted to a sample of heads (heads never interact, so
a sampled oracle is exact for those heads).  Comparisons:
  * planes, metadata, tail ring slots and counters: bit-exact;
  * attention outputs: max |gpu - oracle| <= ATOL (2e-3, fp32 accumulation over dequantized
    values) and, per output row, max |gpu - oracle| / max |oracle| <= RTOL_ROW (1e-3); see
    parity_gate.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import OracleCache
from hierarchical_quantized_kv_amd.binding import Cache
from parity_gate import ATOL, RTOL_ROW, check_close  # noqa: F401 (re-exported)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Lockstep:
    def __init__(self, n_layers, batch, n_heads, head_dim, max_ctx, gamma_max, heads=None,
                 layers=None, draft_offset=8, tag="", meta_fp16=False, split_upper=False):
        self.B, self.H, self.D, self.L = batch, n_heads, head_dim, n_layers
        self.G = 128
        self.heads = list(range(n_heads)) if heads is None else list(heads)
        self.layers = list(range(n_layers)) if layers is None else list(layers)
        self.tag = tag
        self.split_upper = split_upper
        self.gpu = Cache(n_layers, batch, n_heads, head_dim, max_ctx, gamma_max,
                         draft_offset=draft_offset, meta_fp16=meta_fp16, split_upper=split_upper)
        self.orc = {l: OracleCache(1, batch, len(self.heads), head_dim, self.G, max_ctx,
                                   gamma_max, draft_offset, meta_fp16) for l in self.layers}
        self.max_rel = 0.0
        self.max_abs = 0.0

    # inputs arrive as torch fp16 tensors on the GPU ([B][n][H][D] / [B][H][D] / [B][m][H][D])
    def _host_heads(self, t, head_axis):
        idx = torch.as_tensor(self.heads, device=t.device)
        return t.index_select(head_axis, idx).cpu().numpy()

    def append(self, layer, k, v, n=None):
        self.gpu.append(layer, k, v, n)
        if layer in self.orc:
            self.orc[layer].append(0, self._host_heads(k, 2), self._host_heads(v, 2), n)

    def prefill(self, layer, k, v, n=None):
        self.gpu.prefill(layer, k, v, n)
        if layer in self.orc:
            self.orc[layer].prefill(0, self._host_heads(k, 2), self._host_heads(v, 2), n)

    def rollback(self, layer, n_drop):
        self.gpu.rollback(layer, n_drop)
        for l in ([layer] if layer >= 0 else self.layers):
            if l in self.orc:
                self.orc[l].rollback(0, n_drop)

    def flush(self, layer, min_tail=None):
        f = self.gpu.flush(layer, min_tail)
        for l in ([layer] if layer >= 0 else self.layers):
            if l in self.orc:
                fo = self.orc[l].flush(0, min_tail)
                if layer >= 0 or l == self.L - 1:
                    assert np.array_equal(f, fo), (f, fo)
        return f

    def _cmp_out(self, got, ref, what):
        got = got.cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
        mad, rel = check_close(got, ref, f"{self.tag} {what}")
        self.max_abs = max(self.max_abs, mad)
        self.max_rel = max(self.max_rel, rel)
        return mad, rel

    def draft(self, layer, q, sm_scale=1.0):
        out = self.gpu.attend_draft(layer, q, sm_scale)
        if layer in self.orc:
            ref = self.orc[layer].attend_draft(0, self._host_heads(q, 1), sm_scale)
            torch.cuda.synchronize()
            self._cmp_out(out[:, self.heads], ref, f"draft L{layer}")
        return out

    def draft_bits(self, layer, q, bits, sm_scale=1.0):
        out = self.gpu.attend_draft_bits(layer, q, bits, sm_scale)
        if layer in self.orc:
            ref = self.orc[layer].attend_draft_bits(0, self._host_heads(q, 1), bits, sm_scale)
            torch.cuda.synchronize()
            self._cmp_out(out[:, self.heads], ref, f"draft{bits} L{layer}")
        return out

    def verify(self, layer, q, sm_scale=1.0):
        out = self.gpu.attend_verify(layer, q, sm_scale)
        if layer in self.orc:
            ref = self.orc[layer].attend_verify(0, self._host_heads(q, 2), sm_scale)
            torch.cuda.synchronize()
            self._cmp_out(out[:, :, self.heads], ref, f"verify L{layer}")
        return out

    def check_state(self, layer):
        g = self.gpu.state(layer)
        o = self.orc[layer].state(0)
        for a, b, n in zip(g, o, ("nq", "nt", "head")):
            assert np.array_equal(a, b), f"{self.tag} L{layer} {n}: gpu {a} oracle {b}"
        return g

    def check_planes(self, layer):
        """Bit-exact comparison of the live part of every section for the sampled heads."""
        nq, nt, head = self.check_state(layer)
        img = self.orc[layer].export_layer(0)
        if self.split_upper:  # the upper planes as the top and middle 2-bit planes
            img.update(self.orc[layer].export_upper_split(0))
        hs = torch.as_tensor(self.heads, device="cuda")
        G = self.G
        torch.cuda.synchronize()
        for b in range(self.B):
            q = int(nq[b])
            sec = lambda name: self.gpu.section(name, layer)[b].index_select(0, hs)
            # fp16 metadata is compared through its exact fp32 values (the oracle keeps floats)
            host = lambda t: t.float().cpu().numpy() if t.dtype == torch.float16 else t.cpu().numpy()
            upper_k, upper_v = (("tk", "mk"), ("tv", "mv")) if self.split_upper else (("uk",), ("uv",))
            for name, rows in [(n, q) for n in upper_k] + [("lk", q), ("vmeta", q)]:
                got = host(sec(name)[:, :rows])
                ref = img[name][b, :, :rows]
                assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), \
                    f"{self.tag} L{layer} b{b} {name} differs"
            for name in upper_v + ("lv", "kmeta"):
                got = host(sec(name)[:, : q // G])
                ref = img[name][b, :, : q // G]
                assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), \
                    f"{self.tag} L{layer} b{b} {name} differs"
            slots = [(int(head[b]) + i) % (2 * G) for i in range(int(nt[b]))]
            for name in ("tail_k", "tail_v"):
                got = sec(name).cpu().numpy().view(np.uint16)[:, slots]
                ref = img[name][b][:, slots]
                assert np.array_equal(got, ref), f"{self.tag} L{layer} b{b} {name} differs"
