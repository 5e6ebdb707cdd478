"""ctypes binding of libquantspec.so (include/quantspec.h).

Argument marshalling only: torch tensors provide device memory and streams, every step of the
cache runs in the library's HIP kernels.  There is no fallback: if the library is not built,
``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libquantspec.so")

QS_OK, QS_ERR_INVALID_ARG, QS_ERR_CAPACITY, QS_ERR_STATE, QS_ERR_BUFFER, QS_ERR_DEVICE = range(6)
STATUS = {0: "QS_OK", 1: "QS_ERR_INVALID_ARG", 2: "QS_ERR_CAPACITY", 3: "QS_ERR_STATE",
          4: "QS_ERR_BUFFER", 5: "QS_ERR_DEVICE"}

# Every symbol include/quantspec.h declares.
EXPORTS = ("qs_arena_bytes", "qs_arena_layout", "qs_cache_create", "qs_cache_destroy",
           "qs_append", "qs_prefill", "qs_rollback", "qs_flush", "qs_attend_draft",
           "qs_attend_verify", "qs_get_state", "qs_last_error", "qs_spec_workspace_bytes",
           "qs_spec_accept", "qs_state_to_device", "qs_state_from_device", "qs_append_dev",
           "qs_rollback_dev", "qs_flush_dev", "qs_commit_dev", "qs_attend_draft_dev",
           "qs_attend_verify_dev", "qs_append_attend_draft", "qs_append_attend_verify",
           "qs_attend_draft_gqa", "qs_attend_verify_gqa", "qs_attend_draft_bits",
           "qs_spec_accept_static")

# Bits of the device-mode error word (include/quantspec.h, device mode).
DEV_ERR_APPEND, DEV_ERR_ROLLBACK, DEV_ERR_FLUSH, DEV_ERR_ATTEND = 1, 2, 4, 8


class QsConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "batch", "n_heads", "head_dim", "group", "max_ctx", "gamma_max",
        "draft_offset", "meta_fp16", "split_upper")]


class QsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "uk", "lk", "uv", "lv", "kmeta", "vmeta", "tail_k", "tail_v", "work", "state",
        "uk_bytes", "uv_bytes", "kmeta_bytes", "vmeta_bytes", "tail_bytes", "work_bytes",
        "state_bytes", "total")]


class QsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Loads libquantspec.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built: run python -m "
                               "hierarchical_quantized_kv_amd.build_lib (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB)
        P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        PI = ctypes.POINTER(ctypes.c_int32)
        L.qs_arena_bytes.argtypes = [ctypes.POINTER(QsConfig)]
        L.qs_arena_bytes.restype = ctypes.c_size_t
        L.qs_arena_layout.argtypes = [ctypes.POINTER(QsConfig), ctypes.POINTER(QsLayout)]
        L.qs_cache_create.argtypes = [ctypes.POINTER(QsConfig), P, ctypes.c_size_t,
                                      ctypes.POINTER(P)]
        L.qs_cache_destroy.argtypes = [P]
        L.qs_append.argtypes = [P, I32, P, P, I32, PI, P]
        L.qs_prefill.argtypes = [P, I32, P, P, I32, PI, P]
        L.qs_rollback.argtypes = [P, I32, PI]
        L.qs_flush.argtypes = [P, I32, I32, P, PI]
        L.qs_attend_draft.argtypes = [P, I32, P, F, P, P]
        L.qs_attend_verify.argtypes = [P, I32, P, I32, F, P, P]
        L.qs_attend_draft_bits.argtypes = [P, I32, P, I32, F, P, P]
        L.qs_get_state.argtypes = [P, I32, PI, PI, PI]
        L.qs_append_attend_draft.argtypes = [P, I32, P, P, I32, PI, P, F, P, P]
        L.qs_attend_draft_gqa.argtypes = [P, I32, P, I32, F, P, P]
        L.qs_attend_verify_gqa.argtypes = [P, I32, P, I32, I32, F, P, P]
        L.qs_append_attend_verify.argtypes = [P, I32, P, P, P, I32, F, P, P]
        L.qs_last_error.argtypes = [P]
        L.qs_last_error.restype = ctypes.c_char_p
        L.qs_spec_workspace_bytes.argtypes = [I32, I32, I32]
        L.qs_spec_workspace_bytes.restype = ctypes.c_size_t
        L.qs_spec_accept.argtypes = [P, P, P, P, I32, I32, I32, P, ctypes.c_size_t, P, P, P]
        L.qs_spec_accept_static.argtypes = [P, P, P, P, I32, I32, I32, P, P, P]
        L.qs_state_to_device.argtypes = [P, P]
        L.qs_state_from_device.argtypes = [P, P, PI]
        L.qs_append_dev.argtypes = [P, I32, P, P, I32, P]
        L.qs_rollback_dev.argtypes = [P, I32, I32, P, P]
        L.qs_flush_dev.argtypes = [P, I32, I32, P]
        L.qs_commit_dev.argtypes = [P, I32, P]
        L.qs_attend_draft_dev.argtypes = [P, I32, P, F, P, P]
        L.qs_attend_verify_dev.argtypes = [P, I32, P, I32, F, P, P]
        for f in EXPORTS:
            if f not in ("qs_arena_bytes", "qs_last_error", "qs_spec_workspace_bytes"):
                getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _i32(a, n, name="counts"):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
    if arr.shape[0] != n:
        raise ValueError(f"{name}: expected {n} entries, got {arr.shape[0]}")
    return arr


def _ptr_i32(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_config(n_layers, batch, n_heads, head_dim, max_ctx, gamma_max, group=128,
                draft_offset=8, meta_fp16=False, split_upper=False) -> QsConfig:
    return QsConfig(n_layers, batch, n_heads, head_dim, group, max_ctx, gamma_max, draft_offset,
                    int(meta_fp16), int(split_upper))


def arena_layout(cfg: QsConfig) -> QsLayout:
    lay = QsLayout()
    st = lib().qs_arena_layout(ctypes.byref(cfg), ctypes.byref(lay))
    if st != QS_OK:
        raise QsError(st, "invalid configuration")
    return lay


class Cache:
    """A cache over a torch uint8 arena on the current device; verbs mirror the C ABI."""

    def __init__(self, n_layers, batch, n_heads, head_dim, max_ctx, gamma_max, group=128,
                 draft_offset=8, device="cuda", meta_fp16=False, split_upper=False):
        import torch
        self.torch = torch
        self.cfg = make_config(n_layers, batch, n_heads, head_dim, max_ctx, gamma_max, group,
                               draft_offset, meta_fp16, split_upper)
        self.split_upper = bool(split_upper)
        self.L, self.B, self.H, self.D = n_layers, batch, n_heads, head_dim
        self.G, self.T, self.gamma_max = group, max_ctx, gamma_max
        self.meta_fp16 = bool(meta_fp16)
        self.layout = arena_layout(self.cfg)
        nbytes = self.layout.total
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        st = lib().qs_cache_create(ctypes.byref(self.cfg), ctypes.c_void_p(self.arena.data_ptr()),
                                   nbytes, ctypes.byref(h))
        if st != QS_OK:
            raise QsError(st, "qs_cache_create")
        self._h = h
        self._destroy = lib().qs_cache_destroy  # held so that close() still works at shutdown

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _stream(self, stream):
        s = stream if stream is not None else self.torch.cuda.current_stream()
        return ctypes.c_void_p(s.cuda_stream)

    def _check(self, st, what):
        if st != QS_OK:
            raise QsError(st, f"{what}: {lib().qs_last_error(self._h).decode()}")

    def _dev(self, t, dtype, name, shape=None):
        """Device pointer of t after checking that it is a contiguous tensor of dtype (and of
        shape, when given) on the arena's device; raises ValueError otherwise (the kernels
        trust these sizes)."""
        if not isinstance(t, self.torch.Tensor):
            raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
        if t.device != self.arena.device:
            raise ValueError(f"{name}: on {t.device}, the cache's arena is on {self.arena.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        return ctypes.c_void_p(t.data_ptr())

    def _kv(self, k, v, hq=None):
        """k and v: fp16 [B][n][H][D] of the same shape; returns n."""
        if not isinstance(k, self.torch.Tensor) or k.dim() != 4:
            raise ValueError("k: expected a 4-d tensor [B][n][H][D]")
        n = k.shape[1]
        shape = (self.B, n, self.H if hq is None else hq, self.D)
        return n, self._dev(k, self.torch.float16, "k", shape), self._dev(v, self.torch.float16, "v", shape)

    def _out(self, out, shape, device):
        if out is None:
            return self.torch.empty(shape, dtype=self.torch.float32, device=device)
        return out

    def append(self, layer, k, v, n=None, stream=None):
        n_max, pk, pv = self._kv(k, v)
        nn = _i32(n, self.B)
        self._check(lib().qs_append(self._h, layer, pk, pv, n_max, _ptr_i32(nn),
                                    self._stream(stream)), "qs_append")

    def prefill(self, layer, k, v, n=None, stream=None):
        """Bulk "quantize once" of a prompt: k, v fp16 [B][n_max][H][D]."""
        n_max, pk, pv = self._kv(k, v)
        nn = _i32(n, self.B)
        self._check(lib().qs_prefill(self._h, layer, pk, pv, n_max, _ptr_i32(nn),
                                     self._stream(stream)), "qs_prefill")

    def rollback(self, layer, n_drop):
        nd = _i32(n_drop, self.B, "n_drop")
        self._check(lib().qs_rollback(self._h, layer, _ptr_i32(nd)), "qs_rollback")

    def flush(self, layer=-1, min_tail=None, stream=None):
        flushed = np.zeros(self.B, dtype=np.int32)
        self._check(lib().qs_flush(self._h, layer, self.G if min_tail is None else min_tail,
                                   self._stream(stream), _ptr_i32(flushed)), "qs_flush")
        return flushed

    def attend_draft(self, layer, q, sm_scale=1.0, out=None, stream=None):
        torch = self.torch
        shape = (self.B, self.H, self.D)
        pq = self._dev(q, torch.float16, "q", shape)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_attend_draft(self._h, layer, pq, float(sm_scale),
                                          self._dev(out, torch.float32, "out", shape),
                                          self._stream(stream)), "qs_attend_draft")
        return out

    def _verify_q(self, q, hq=None):
        if not isinstance(q, self.torch.Tensor) or q.dim() != 4:
            raise ValueError("q: expected a 4-d tensor [B][m][H][D]")
        shape = (self.B, q.shape[1], self.H if hq is None else hq, self.D)
        return shape, self._dev(q, self.torch.float16, "q", shape)

    def attend_draft_bits(self, layer, q, bits, sm_scale=1.0, out=None, stream=None):
        """Draft on the top `bits` (4, or 2 with split_upper) bits of every code."""
        torch = self.torch
        shape = (self.B, self.H, self.D)
        pq = self._dev(q, torch.float16, "q", shape)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_attend_draft_bits(self._h, layer, pq, int(bits), float(sm_scale),
                                               self._dev(out, torch.float32, "out", shape),
                                               self._stream(stream)), "qs_attend_draft_bits")
        return out

    def attend_verify(self, layer, q, sm_scale=1.0, out=None, stream=None):
        torch = self.torch
        shape, pq = self._verify_q(q)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_attend_verify(self._h, layer, pq, shape[1], float(sm_scale),
                                           self._dev(out, torch.float32, "out", shape),
                                           self._stream(stream)), "qs_attend_verify")
        return out

    def attend_draft_gqa(self, layer, q, g, sm_scale=1.0, out=None, stream=None):
        """Grouped queries: q fp16 [B][H*g][D] (query head h*g + r reads cached head h)."""
        torch = self.torch
        g = int(g)
        shape = (self.B, self.H * g, self.D)
        pq = self._dev(q, torch.float16, "q", shape)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_attend_draft_gqa(self._h, layer, pq, g, float(sm_scale),
                                              self._dev(out, torch.float32, "out", shape),
                                              self._stream(stream)), "qs_attend_draft_gqa")
        return out

    def attend_verify_gqa(self, layer, q, g, sm_scale=1.0, out=None, stream=None):
        """Grouped queries: q fp16 [B][m][H*g][D]."""
        torch = self.torch
        g = int(g)
        shape, pq = self._verify_q(q, self.H * g)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_attend_verify_gqa(self._h, layer, pq, shape[1], g, float(sm_scale),
                                               self._dev(out, torch.float32, "out", shape),
                                               self._stream(stream)), "qs_attend_verify_gqa")
        return out

    def append_attend_draft(self, layer, k, v, q, n=None, sm_scale=1.0, out=None, stream=None):
        """append(layer, k, v, n) then attend_draft(layer, q), fused into one launch pair."""
        torch = self.torch
        n_max, pk, pv = self._kv(k, v)
        shape = (self.B, self.H, self.D)
        pq = self._dev(q, torch.float16, "q", shape)
        out = self._out(out, shape, q.device)
        nn = _i32(n, self.B)
        self._check(lib().qs_append_attend_draft(
            self._h, layer, pk, pv, n_max, _ptr_i32(nn), pq, float(sm_scale),
            self._dev(out, torch.float32, "out", shape), self._stream(stream)),
            "qs_append_attend_draft")
        return out

    def append_attend_verify(self, layer, k, v, q, sm_scale=1.0, out=None, stream=None):
        """append(layer, k, v) of the m verified tokens then attend_verify(layer, q), fused."""
        torch = self.torch
        shape, pq = self._verify_q(q)
        pk = self._dev(k, torch.float16, "k", shape)
        pv = self._dev(v, torch.float16, "v", shape)
        out = self._out(out, shape, q.device)
        self._check(lib().qs_append_attend_verify(
            self._h, layer, pk, pv, pq, shape[1], float(sm_scale),
            self._dev(out, torch.float32, "out", shape), self._stream(stream)),
            "qs_append_attend_verify")
        return out

    def state(self, layer):
        nq = np.zeros(self.B, np.int32)
        nt = np.zeros(self.B, np.int32)
        hd = np.zeros(self.B, np.int32)
        self._check(lib().qs_get_state(self._h, layer, _ptr_i32(nq), _ptr_i32(nt), _ptr_i32(hd)),
                    "qs_get_state")
        return nq, nt, hd

    # ---- device mode: the counters in device memory; the _dev verbs only enqueue kernels,
    # so a sequence of them can be captured in a graph and replayed ------------------------
    def to_device_state(self, stream=None):
        self._check(lib().qs_state_to_device(self._h, self._stream(stream)), "qs_state_to_device")

    def from_device_state(self, stream=None) -> int:
        """Back to host mode; returns the device error word (DEV_ERR_* bits)."""
        err = np.zeros(1, np.int32)
        self._check(lib().qs_state_from_device(self._h, self._stream(stream), _ptr_i32(err)),
                    "qs_state_from_device")
        return int(err[0])

    def append_dev(self, layer, k, v, stream=None):
        n_max, pk, pv = self._kv(k, v)
        self._check(lib().qs_append_dev(self._h, layer, pk, pv, n_max, self._stream(stream)),
                    "qs_append_dev")

    def rollback_dev(self, layer, n, sub=None, stream=None):
        """Drops n - sub[b] tail tokens of each sequence b (sub: device int32 [B] or None; it
        must keep its values until the rollback is committed)."""
        p = None
        if sub is not None:
            p = self._dev(sub, self.torch.int32, "sub", (self.B,))
        self._check(lib().qs_rollback_dev(self._h, layer, int(n), p, self._stream(stream)),
                    "qs_rollback_dev")

    def flush_dev(self, layer=-1, min_tail=None, stream=None):
        self._check(lib().qs_flush_dev(self._h, layer, self.G if min_tail is None else min_tail,
                                       self._stream(stream)), "qs_flush_dev")

    def commit_dev(self, layer=-1, stream=None):
        self._check(lib().qs_commit_dev(self._h, layer, self._stream(stream)), "qs_commit_dev")

    def attend_draft_dev(self, layer, q, out, sm_scale=1.0, stream=None):
        torch = self.torch
        shape = (self.B, self.H, self.D)
        self._check(lib().qs_attend_draft_dev(self._h, layer, self._dev(q, torch.float16, "q", shape),
                                              float(sm_scale),
                                              self._dev(out, torch.float32, "out", shape),
                                              self._stream(stream)), "qs_attend_draft_dev")

    def attend_verify_dev(self, layer, q, out, sm_scale=1.0, stream=None):
        torch = self.torch
        shape, pq = self._verify_q(q)
        self._check(lib().qs_attend_verify_dev(self._h, layer, pq, shape[1], float(sm_scale),
                                               self._dev(out, torch.float32, "out", shape),
                                               self._stream(stream)), "qs_attend_verify_dev")

    # ---- views of the arena (layout of include/quantspec.h), for inspection -------------
    def section(self, name, layer):
        """Device view of one layer of an arena section, shaped as the header documents."""
        torch = self.torch
        B, H, T, D, G = self.B, self.H, self.T, self.D, self.G
        NG = T // G
        lay = self.layout
        mt = torch.float16 if self.meta_fp16 else torch.float32  # (scale, offset) or (scale, zero)
        shapes = {
            "uk": (torch.uint8, lay.uk, (B, H, T, D // 2)),
            "lk": (torch.uint8, lay.lk, (B, H, T, D // 2)),
            "uv": (torch.uint8, lay.uv, (B, H, NG, 2, D, G // 4)),
            "lv": (torch.uint8, lay.lv, (B, H, NG, 2, D, G // 4)),
            "kmeta": (mt, lay.kmeta, (B, H, NG, D, 2)),
            "vmeta": (mt, lay.vmeta, (B, H, T, 2)),
            "tail_k": (torch.float16, lay.tail_k, (B, H, 2 * G, D)),
            "tail_v": (torch.float16, lay.tail_v, (B, H, 2 * G, D)),
        }
        if name in ("tk", "mk", "tv", "mv"):
            # split-upper layout: the C_T (top) and C_M (middle) 2-bit planes are the first and
            # second halves of each (sequence, head) stripe of uk (keys) and uv (values)
            if not self.split_upper:
                raise ValueError(f"section {name}: the cache does not use the split-upper layout")
            off, shape = ((lay.uk, (B, H, 2, T, D // 4)) if name[1] == "k"
                          else (lay.uv, (B, H, 2, NG, 2, D, G // 8)))
            n = int(np.prod(shape))
            view = self.arena[off + layer * n:off + (layer + 1) * n].view(*shape)
            return view[:, :, 0] if name[0] == "t" else view[:, :, 1]
        dtype, off, shape = shapes[name]
        esize = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape))
        start = off + layer * n * esize
        return self.arena[start:start + n * esize].view(dtype).view(*shape)


def spec_workspace_bytes(batch: int, gamma: int, vocab: int) -> int:
    """Workspace qs_spec_accept needs (qs_spec_workspace_bytes); 0 for arguments it rejects."""
    return int(lib().qs_spec_workspace_bytes(batch, gamma, vocab))


def spec_accept(target_logits, draft_logits, draft_tokens, uniforms, workspace=None, stream=None,
                n_out=None, next_out=None):
    """Speculative accept / correct on the GPU (qs_spec_accept).  target_logits fp32
    [B][gamma+1][V], draft_logits fp32 [B][gamma][V], draft_tokens int32 [B][gamma], uniforms fp32
    [B][gamma+1], all on the device.  Returns device int32 tensors (n_accepted, next_token),
    written into n_out / next_out when given."""
    import torch
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    for t, dt, shape, name in ((target_logits, torch.float32, (B, gamma + 1, V), "target_logits"),
                               (draft_logits, torch.float32, (B, gamma, V), "draft_logits"),
                               (draft_tokens, torch.int32, (B, gamma), "draft_tokens"),
                               (uniforms, torch.float32, (B, gamma + 1), "uniforms")):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous() and tuple(t.shape) == shape):
            raise ValueError(f"{name}: expected a contiguous {dt} device tensor of shape {shape}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")
        if t.device != target_logits.device:
            raise ValueError(f"{name}: on {t.device}, target_logits on {target_logits.device}")
    need = spec_workspace_bytes(B, gamma, V)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=target_logits.device)
    elif not (workspace.is_cuda and workspace.is_contiguous()
              and workspace.device == target_logits.device):
        raise ValueError("workspace: expected a contiguous device tensor on "
                         f"{target_logits.device}")
    n = torch.empty(B, dtype=torch.int32, device=target_logits.device) if n_out is None else n_out
    nxt = (torch.empty(B, dtype=torch.int32, device=target_logits.device) if next_out is None
           else next_out)
    for t, name in ((n, "n_out"), (nxt, "next_out")):
        if not (t.is_cuda and t.dtype == torch.int32 and t.is_contiguous() and t.numel() == B
                and t.device == target_logits.device):
            raise ValueError(f"{name}: expected a contiguous int32 tensor of {B} entries on "
                             f"{target_logits.device}")
    s = stream if stream is not None else torch.cuda.current_stream()
    P = ctypes.c_void_p
    st = lib().qs_spec_accept(P(target_logits.data_ptr()), P(draft_logits.data_ptr()),
                              P(draft_tokens.data_ptr()), P(uniforms.data_ptr()), B, gamma, V,
                              P(workspace.data_ptr()), workspace.numel() * workspace.element_size(), P(n.data_ptr()),
                              P(nxt.data_ptr()), P(s.cuda_stream))
    if st != QS_OK:
        raise QsError(st, "qs_spec_accept")
    return n, nxt


SPEC_STATIC_BYTES = 4 << 20  # the library's own workspace of qs_spec_accept_static, per GPU


def spec_accept_static(target_logits, draft_logits, draft_tokens, uniforms, n_out, next_out,
                       stream=None):
    """qs_spec_accept_static: the accept / correct step with the library's device-resident
    workspace, for callers that cannot allocate (graph capture).  Same tensors as spec_accept;
    the outputs n_out / next_out (device int32 [B]) must be given."""
    import torch
    B, g1, V = target_logits.shape
    gamma = g1 - 1
    for t, dt, shape, name in ((target_logits, torch.float32, (B, gamma + 1, V), "target_logits"),
                               (draft_logits, torch.float32, (B, gamma, V), "draft_logits"),
                               (draft_tokens, torch.int32, (B, gamma), "draft_tokens"),
                               (uniforms, torch.float32, (B, gamma + 1), "uniforms"),
                               (n_out, torch.int32, (B,), "n_out"),
                               (next_out, torch.int32, (B,), "next_out")):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous() and tuple(t.shape) == shape
                and t.device == target_logits.device):
            raise ValueError(f"{name}: expected a contiguous {dt} tensor of shape {shape} on "
                             f"{target_logits.device}")
    s = stream if stream is not None else torch.cuda.current_stream()
    P = ctypes.c_void_p
    st = lib().qs_spec_accept_static(P(target_logits.data_ptr()), P(draft_logits.data_ptr()),
                                     P(draft_tokens.data_ptr()), P(uniforms.data_ptr()), B, gamma,
                                     V, P(n_out.data_ptr()), P(next_out.data_ptr()),
                                     P(s.cuda_stream))
    if st != QS_OK:
        raise QsError(st, "qs_spec_accept_static")

