"""CPU oracle of the hierarchical INT8 KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU library never loads it and shares no code with it; the product path
fails loudly when its HIP extension is missing instead of falling back here.

The arithmetic lives in ``qs_oracle.c`` (plain C, fp32 quantizer, fp64 attention); this module
only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qs_oracle.c")
LIB = os.path.join(HERE, "libqs_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_half_to_float.restype = ctypes.c_float
        L.orc_quantize_group.argtypes = [P, i, i, P, P, P, i]
        L.orc_quantize_group.restype = None
        L.orc_dequant_full.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float]
        L.orc_dequant_full.restype = ctypes.c_double
        L.orc_dequant_upper.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float, i]
        L.orc_dequant_upper.restype = ctypes.c_double
        L.orc_dequant_topk.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float, i, i]
        L.orc_dequant_topk.restype = ctypes.c_double
        L.orc_dequant16_topk.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float, i, i]
        L.orc_dequant16_topk.restype = ctypes.c_double
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_meta16.argtypes = [ctypes.c_float, ctypes.c_float, P, P]
        L.orc_meta16.restype = None
        L.orc_dequant16_full.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float]
        L.orc_dequant16_full.restype = ctypes.c_double
        L.orc_dequant16_upper.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float, i]
        L.orc_dequant16_upper.restype = ctypes.c_double
        L.orc_create.argtypes = [i, i, i, i, i, i, i, i, i]
        L.orc_create.restype = P
        L.orc_destroy.argtypes = [P]
        L.orc_destroy.restype = None
        L.orc_append.argtypes = [P, i, P, P, i, P]
        L.orc_prefill.argtypes = [P, i, P, P, i, P]
        L.orc_spec_accept.argtypes = [P, P, P, P, i, i, i, P, P, P]
        L.orc_rollback.argtypes = [P, i, P]
        L.orc_flush.argtypes = [P, i, i, P]
        L.orc_attend_draft.argtypes = [P, i, P, ctypes.c_double, P]
        L.orc_attend_draft_bits.argtypes = [P, i, P, i, ctypes.c_double, P]
        L.orc_attend_verify.argtypes = [P, i, P, i, ctypes.c_double, P]
        L.orc_get_state.argtypes = [P, i, P, P, P]
        L.orc_read_codes.argtypes = [P, i, i, i, i, P]
        L.orc_set_lower_nibbles.argtypes = [P, i, i]
        L.orc_set_low_bits.argtypes = [P, i, i, i]
        L.orc_export_upper_split.argtypes = [P, i, P, P, P, P]
        L.orc_read_meta.argtypes = [P, i, i, i, P, P]
        L.orc_export_layer.argtypes = [P, i, P, P, P, P, P, P, P, P]
        for f in ("orc_append", "orc_prefill", "orc_spec_accept", "orc_rollback", "orc_flush", "orc_attend_draft",
                  "orc_attend_verify", "orc_get_state", "orc_read_codes", "orc_read_meta",
                  "orc_export_layer", "orc_set_lower_nibbles", "orc_attend_draft_bits",
                  "orc_set_low_bits", "orc_export_upper_split"):
            getattr(L, f).restype = i
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


def _i32(a) -> np.ndarray | None:
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} returned status {code}")
        self.code = code


def quantize_group(x: np.ndarray):
    """Quantizes one group (1-D fp16 array). Returns (scale, zero, codes)."""
    x = _bits16(np.ascontiguousarray(x, dtype=np.float16))
    s = ctypes.c_float()
    z = ctypes.c_float()
    c = np.zeros(x.shape[0], dtype=np.uint8)
    lib().orc_quantize_group(_ptr(x), x.shape[0], 1, ctypes.byref(s), ctypes.byref(z), _ptr(c), 1)
    return s.value, z.value, c


def dequant_full(c8: int, s: float, z: float) -> float:
    return lib().orc_dequant_full(int(c8), float(s), float(z))


def dequant_upper(cu: int, s: float, z: float, off: int) -> float:
    return lib().orc_dequant_upper(int(cu), float(s), float(z), int(off))


def dequant_topk(c8: int, s: float, z: float, k: int, off: int) -> float:
    return lib().orc_dequant_topk(int(c8), float(s), float(z), int(k), int(off))


def dequant16_topk(c8: int, s: float, b: float, k: int, off: int) -> float:
    return lib().orc_dequant16_topk(int(c8), float(s), float(b), int(k), int(off))


def float_to_half(x: float) -> int:
    """Bits of the binary16 nearest to the fp32 value x (ties to even)."""
    return int(lib().orc_float_to_half(float(x)))


def meta16(s: float, z: float):
    """fp16 metadata (scale, offset) of fp32 (s, z), as floats."""
    a, b = ctypes.c_float(), ctypes.c_float()
    lib().orc_meta16(float(s), float(z), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def dequant16_full(c8: int, s: float, b: float) -> float:
    return lib().orc_dequant16_full(int(c8), float(s), float(b))


def dequant16_upper(cu: int, s: float, b: float, off: int) -> float:
    return lib().orc_dequant16_upper(int(cu), float(s), float(b), int(off))


def spec_accept(target_logits, draft_logits, draft_tokens, uniforms):
    """Speculative accept / correct in fp64 (orc_spec_accept).  Shapes: [B][gamma+1][V],
    [B][gamma][V], [B][gamma], [B][gamma+1].  Returns (n_accepted, next_token, margin)."""
    t = np.ascontiguousarray(target_logits, dtype=np.float32)
    d = np.ascontiguousarray(draft_logits, dtype=np.float32)
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B, g1, V = t.shape
    gamma = g1 - 1
    assert d.shape == (B, gamma, V) and x.shape == (B, gamma) and u.shape == (B, gamma + 1)
    n = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    mg = np.zeros(B, np.float64)
    rc = lib().orc_spec_accept(_ptr(t), _ptr(d), _ptr(x), _ptr(u), B, gamma, V, _ptr(n),
                               _ptr(nxt), _ptr(mg))
    if rc != 0:
        raise OracleError(rc, "spec_accept")
    return n, nxt, mg


class OracleCache:
    """The oracle's cache: same verbs as the C ABI, on host memory."""

    def __init__(self, n_layers, batch, n_heads, head_dim, group=128, max_ctx=1024,
                 gamma_max=6, draft_offset=8, meta_fp16=False):
        self.L, self.B, self.H, self.D = n_layers, batch, n_heads, head_dim
        self.G, self.T, self.gamma_max, self.off = group, max_ctx, gamma_max, draft_offset
        self.meta_fp16 = bool(meta_fp16)
        self._h = lib().orc_create(n_layers, batch, n_heads, head_dim, group, max_ctx, gamma_max,
                                   draft_offset, int(self.meta_fp16))
        if not self._h:
            raise OracleError(1, "create")

    def close(self):
        if self._h:
            lib().orc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, rc, what):
        if rc != 0:
            raise OracleError(rc, what)

    def append(self, layer, k, v, n=None):
        k = _bits16(k)
        v = _bits16(v)
        assert k.shape == v.shape and k.shape[0] == self.B and k.shape[2:] == (self.H, self.D)
        self._check(lib().orc_append(self._h, layer, _ptr(k), _ptr(v), k.shape[1],
                                     _ptr(_i32(n))), "append")

    def prefill(self, layer, k, v, n=None):
        k = _bits16(k)
        v = _bits16(v)
        assert k.shape == v.shape and k.shape[0] == self.B and k.shape[2:] == (self.H, self.D)
        self._check(lib().orc_prefill(self._h, layer, _ptr(k), _ptr(v), k.shape[1],
                                      _ptr(_i32(n))), "prefill")

    def rollback(self, layer, n_drop):
        self._check(lib().orc_rollback(self._h, layer, _ptr(_i32(n_drop))), "rollback")

    def flush(self, layer, min_tail=None):
        flushed = np.zeros(self.B, dtype=np.int32)
        self._check(lib().orc_flush(self._h, layer, self.G if min_tail is None else min_tail,
                                    _ptr(flushed)), "flush")
        return flushed

    def attend_draft(self, layer, q, sm_scale=1.0):
        q = _bits16(q)
        assert q.shape == (self.B, self.H, self.D)
        out = np.zeros((self.B, self.H, self.D), dtype=np.float32)
        self._check(lib().orc_attend_draft(self._h, layer, _ptr(q), float(sm_scale), _ptr(out)),
                    "attend_draft")
        return out

    def attend_draft_bits(self, layer, q, bits, sm_scale=1.0):
        """Draft pass on the top `bits` bits of every code (4: attend_draft; 8: the verify
        dequantization)."""
        q = _bits16(q)
        assert q.shape == (self.B, self.H, self.D)
        out = np.zeros((self.B, self.H, self.D), dtype=np.float32)
        self._check(lib().orc_attend_draft_bits(self._h, layer, _ptr(q), int(bits), float(sm_scale),
                                                _ptr(out)), "attend_draft_bits")
        return out

    def attend_verify(self, layer, q, sm_scale=1.0):
        q = _bits16(q)
        assert q.shape[0] == self.B and q.shape[2:] == (self.H, self.D)
        m = q.shape[1]
        out = np.zeros((self.B, m, self.H, self.D), dtype=np.float32)
        self._check(lib().orc_attend_verify(self._h, layer, _ptr(q), m, float(sm_scale),
                                            _ptr(out)), "attend_verify")
        return out

    def state(self, layer):
        nq = np.zeros(self.B, dtype=np.int32)
        nt = np.zeros(self.B, dtype=np.int32)
        hd = np.zeros(self.B, dtype=np.int32)
        self._check(lib().orc_get_state(self._h, layer, _ptr(nq), _ptr(nt), _ptr(hd)), "state")
        return nq, nt, hd

    def set_lower_nibbles(self, layer, value):
        """Test support: every stored code of `layer` gets lower nibble `value`."""
        self._check(lib().orc_set_lower_nibbles(self._h, layer, int(value)), "set_lower_nibbles")

    def set_low_bits(self, layer, nbits, value):
        """Test support: the low `nbits` bits of every stored code of `layer` become `value`."""
        self._check(lib().orc_set_low_bits(self._h, layer, int(nbits), int(value)), "set_low_bits")

    def export_upper_split(self, layer):
        """The split-upper layout's 2-bit planes of one layer (orc_export_upper_split): top
        bits and middle bits, keys [B][H][T][D/4] and values [B][H][NG][2][D][G/8]."""
        B, H, T, D, G = self.B, self.H, self.T, self.D, self.G
        NG = T // G
        out = dict(tk=np.zeros((B, H, T, D // 4), np.uint8), mk=np.zeros((B, H, T, D // 4), np.uint8),
                   tv=np.zeros((B, H, NG, 2, D, G // 8), np.uint8),
                   mv=np.zeros((B, H, NG, 2, D, G // 8), np.uint8))
        self._check(lib().orc_export_upper_split(self._h, layer, *(_ptr(out[k]) for k in
                                                                    ("tk", "mk", "tv", "mv"))),
                    "export_upper_split")
        return out

    def codes(self, layer, b, h, which_v=False):
        out = np.zeros((self.T, self.D), dtype=np.uint8)
        self._check(lib().orc_read_codes(self._h, layer, b, h, int(which_v), _ptr(out)), "codes")
        return out

    def meta(self, layer, b, h):
        km = np.zeros((self.T // self.G, self.D, 2), dtype=np.float32)
        vm = np.zeros((self.T, 2), dtype=np.float32)
        self._check(lib().orc_read_meta(self._h, layer, b, h, _ptr(km), _ptr(vm)), "meta")
        return km, vm

    def export_layer(self, layer):
        """Arena-layout images of one layer (see orc_export_layer)."""
        B, H, T, D, G = self.B, self.H, self.T, self.D, self.G
        NG = T // G
        out = dict(
            uk=np.zeros((B, H, T, D // 2), np.uint8), lk=np.zeros((B, H, T, D // 2), np.uint8),
            uv=np.zeros((B, H, NG, 2, D, G // 4), np.uint8),
            lv=np.zeros((B, H, NG, 2, D, G // 4), np.uint8),
            kmeta=np.zeros((B, H, NG, D, 2), np.float32), vmeta=np.zeros((B, H, T, 2), np.float32),
            tail_k=np.zeros((B, H, 2 * G, D), np.uint16),
            tail_v=np.zeros((B, H, 2 * G, D), np.uint16))
        self._check(lib().orc_export_layer(
            self._h, layer, *(_ptr(out[k]) for k in
                              ("uk", "lk", "uv", "lv", "kmeta", "vmeta", "tail_k", "tail_v"))),
            "export")
        return out
