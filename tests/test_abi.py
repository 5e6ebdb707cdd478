"""The C-ABI library on the CPU: it loads, exports every symbol include/quantspec.h declares, and
its host-only paths (sizes, layout, argument validation before any launch) behave as documented.
No call here reaches the device."""
import ctypes
import os
import re
import subprocess

import pytest

from hierarchical_quantized_kv_amd import binding
from hierarchical_quantized_kv_amd.binding import QsConfig, QsLayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
G = 128


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(qs_\w+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB):
        pytest.fail("libquantspec.so is not built (run __graft_entry__.build())")
    return binding.lib()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert decl == set(binding.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\b(qs_\w+)\b", nm))
    assert decl <= exported, decl - exported
    for name in decl:
        getattr(lib, name)


def cfg(**kw):
    base = dict(n_layers=2, batch=3, n_heads=4, head_dim=128, group=G, max_ctx=8 * G,
                gamma_max=6, draft_offset=8, meta_fp16=0, split_upper=0)
    base.update(kw)
    return QsConfig(*[base[f] for f, _ in QsConfig._fields_])


def test_arena_size_and_layout(lib):
    c = cfg()
    n = lib.qs_arena_bytes(ctypes.byref(c))
    lay = QsLayout()
    assert lib.qs_arena_layout(ctypes.byref(c), ctypes.byref(lay)) == 0
    assert n == lay.total > 0
    offs = [lay.uk, lay.lk, lay.uv, lay.lv, lay.kmeta, lay.vmeta, lay.tail_k, lay.tail_v, lay.work,
            lay.state]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.state + lay.state_bytes == lay.total and lay.state_bytes >= (2 * 3 * 4 + 1) * 4
    lbh = 2 * 3 * 4
    assert lay.uk_bytes == lbh * 8 * G * 64 and lay.uv_bytes == lbh * 8 * 128 * 64
    assert lay.kmeta_bytes == lbh * 8 * 128 * 8 and lay.vmeta_bytes == lbh * 8 * G * 8
    # fp16 metadata: half the metadata bytes, every other section the same size
    lay16 = QsLayout()
    assert lib.qs_arena_layout(ctypes.byref(cfg(meta_fp16=1)), ctypes.byref(lay16)) == 0
    assert lay16.kmeta_bytes == lay.kmeta_bytes // 2 and lay16.vmeta_bytes == lay.vmeta_bytes // 2
    for f in ("uk_bytes", "uv_bytes", "tail_bytes", "work_bytes", "state_bytes"):
        assert getattr(lay16, f) == getattr(lay, f)
    for bad in (cfg(head_dim=96), cfg(group=64), cfg(max_ctx=100), cfg(batch=0),
                cfg(batch=65), cfg(gamma_max=15 + 1), cfg(draft_offset=4), cfg(meta_fp16=2)):
        assert lib.qs_arena_bytes(ctypes.byref(bad)) == 0
        assert lib.qs_arena_layout(ctypes.byref(bad), ctypes.byref(lay)) == binding.QS_ERR_INVALID_ARG


FAKE = 1 << 40   # an aligned address that is never dereferenced by host-only paths


def create(lib, c):
    h = ctypes.c_void_p()
    n = lib.qs_arena_bytes(ctypes.byref(c))
    st = lib.qs_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE), n, ctypes.byref(h))
    assert st == 0
    return h


def test_create_checks_arena(lib):
    c = cfg()
    n = lib.qs_arena_bytes(ctypes.byref(c))
    h = ctypes.c_void_p()
    assert lib.qs_cache_create(ctypes.byref(c), None, n, ctypes.byref(h)) == binding.QS_ERR_BUFFER
    assert lib.qs_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE + 64), n,
                               ctypes.byref(h)) == binding.QS_ERR_BUFFER
    assert lib.qs_cache_create(ctypes.byref(c), ctypes.c_void_p(FAKE), n - 1,
                               ctypes.byref(h)) == binding.QS_ERR_BUFFER
    bad = cfg(head_dim=80)
    assert lib.qs_cache_create(ctypes.byref(bad), ctypes.c_void_p(FAKE), n,
                               ctypes.byref(h)) == binding.QS_ERR_INVALID_ARG
    h = create(lib, c)
    assert lib.qs_cache_destroy(h) == 0
    assert lib.qs_cache_destroy(None) == 0


def arr(*v):
    return (ctypes.c_int32 * len(v))(*v)


def test_validation_before_any_launch(lib):
    c = cfg()
    h = create(lib, c)
    P = ctypes.c_void_p(FAKE)
    # counters start empty
    nq, nt, hd = arr(9, 9, 9), arr(9, 9, 9), arr(9, 9, 9)
    assert lib.qs_get_state(h, 1, nq, nt, hd) == 0
    assert list(nq) == list(nt) == list(hd) == [0, 0, 0]
    assert lib.qs_get_state(h, 2, nq, nt, hd) == binding.QS_ERR_INVALID_ARG
    # append: bad layer, null tensors, n > n_max, ring overflow -- all rejected before launch
    assert lib.qs_append(h, 2, P, P, 1, None, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_append(h, 0, None, P, 1, None, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_append(h, 0, P, P, 4, arr(1, 5, 0), None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_append(h, 0, P, P, 2 * G + 1, None, None) == binding.QS_ERR_CAPACITY
    assert b"overflow" in lib.qs_last_error(h)
    # prefill: bad layer, null tensors, n > n_max, past max_ctx, n_max / G too large; n = 0 is a
    # no-op that launches nothing
    assert lib.qs_prefill(h, 2, P, P, 1, None, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_prefill(h, 0, P, None, 1, None, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_prefill(h, 0, P, P, 4, arr(1, 5, 0), None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_prefill(h, 0, P, P, 9 * G, None, None) == binding.QS_ERR_CAPACITY
    assert b"max_ctx" in lib.qs_last_error(h)
    assert lib.qs_prefill(h, 0, P, P, 65536 * G, arr(0, 0, 0), None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_prefill(h, 0, P, P, 0, None, None) == 0
    # rollback of an empty tail
    assert lib.qs_rollback(h, -1, arr(0, 1, 0)) == binding.QS_ERR_STATE
    assert lib.qs_rollback(h, 0, arr(0, 0, -1)) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_rollback(h, -1, arr(0, 0, 0)) == 0
    assert lib.qs_rollback(h, 0, None) == 0
    # flush: nothing selected launches nothing; min_tail > 2G rejected
    fl = arr(7, 7, 7)
    assert lib.qs_flush(h, -1, G, None, fl) == 0 and list(fl) == [0, 0, 0]
    assert lib.qs_flush(h, 0, 2 * G + 1, None, fl) == binding.QS_ERR_INVALID_ARG
    # attention over empty sequences, bad m, bad scale
    assert lib.qs_attend_draft(h, 0, P, ctypes.c_float(1.0), P, None) == binding.QS_ERR_STATE
    assert lib.qs_attend_verify(h, 0, P, 0, ctypes.c_float(1.0), P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_verify(h, 0, P, 8, ctypes.c_float(1.0), P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_verify(h, 0, P, 1, ctypes.c_float(1.0), P, None) == binding.QS_ERR_STATE
    assert lib.qs_attend_draft(h, 0, P, ctypes.c_float(float("nan")), P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_draft(h, 0, None, ctypes.c_float(1.0), P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_get_state(h, 0, nq, nt, hd) == 0 and list(nt) == [0, 0, 0]
    # grouped queries: g in 1..16, m * g within gamma_max + 1 = 7 query columns per head
    F1 = ctypes.c_float(1.0)
    assert lib.qs_attend_draft_gqa(h, 0, P, 0, F1, P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_draft_gqa(h, 0, P, 8, F1, P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_verify_gqa(h, 0, P, 2, 4, F1, P, None) == binding.QS_ERR_INVALID_ARG
    assert lib.qs_attend_draft_gqa(h, 0, P, 7, F1, P, None) == binding.QS_ERR_STATE  # empty
    assert lib.qs_attend_verify_gqa(h, 0, P, 1, 7, F1, P, None) == binding.QS_ERR_STATE
    lib.qs_cache_destroy(h)


def test_device_mode_verbs_rejected_in_host_mode(lib):
    """Before qs_state_to_device the _dev verbs (and qs_state_from_device) return QS_ERR_STATE
    without launching anything; host verbs keep working."""
    h = create(lib, cfg())
    P = ctypes.c_void_p(FAKE)
    F1 = ctypes.c_float(1.0)
    err = arr(0)
    for st in (lib.qs_state_from_device(h, None, err),
               lib.qs_append_dev(h, 0, P, P, 1, None),
               lib.qs_rollback_dev(h, -1, 1, None, None),
               lib.qs_flush_dev(h, -1, G, None),
               lib.qs_commit_dev(h, -1, None),
               lib.qs_attend_draft_dev(h, 0, P, F1, P, None),
               lib.qs_attend_verify_dev(h, 0, P, 2, F1, P, None)):
        assert st == binding.QS_ERR_STATE
        assert b"device mode" in lib.qs_last_error(h)
    assert lib.qs_rollback(h, -1, arr(0, 0, 0)) == 0
    lib.qs_cache_destroy(h)


def test_spec_accept_validation_before_any_launch(lib):
    P = ctypes.c_void_p(FAKE)
    # per sequence, fp32: (max, sum) of each of the 2 gamma + 1 rows per 4096-token part, (max,
    # 1/sum) per row, the two sampling totals of the rejection point per part, gamma acceptance
    # ratios and the target and draft logits of the gamma drafted tokens
    ws_bytes = lambda B, g, parts: B * (2 * (2 * g + 1) * parts + 2 * (2 * g + 1)
                                        + 2 * parts + g + 2 * g) * 4
    assert lib.qs_spec_workspace_bytes(2, 6, 100) == ws_bytes(2, 6, 1)       # one part
    assert lib.qs_spec_workspace_bytes(2, 6, 32000) == ws_bytes(2, 6, 8)     # eight parts
    assert lib.qs_spec_workspace_bytes(1, 15, 1 << 20) == ws_bytes(1, 15, 256)
    for args in ((0, 6, 100), (65536, 6, 100), (1, 16, 100), (1, 6, 0), (1, 6, (1 << 20) + 1)):
        assert lib.qs_spec_workspace_bytes(*args) == 0, args
    ws = lib.qs_spec_workspace_bytes(2, 6, 100)
    call = lambda *a: lib.qs_spec_accept(*a)
    ok = (P, P, P, P, 2, 6, 100, P, ws, P, P, None)
    for i in (0, 1, 2, 3, 7, 9, 10):                     # every pointer is required
        args = list(ok)
        args[i] = None
        assert call(*args) == binding.QS_ERR_INVALID_ARG, i
    for b_, g_, v_ in ((0, 6, 100), (65536, 6, 100), (2, 0, 100), (2, 16, 100), (2, 6, 0),
                       (2, 6, (1 << 20) + 1)):
        assert call(P, P, P, P, b_, g_, v_, P, 1 << 20, P, P, None) == binding.QS_ERR_INVALID_ARG
    assert call(P, P, P, P, 2, 6, 100, P, ws - 1, P, P, None) == binding.QS_ERR_BUFFER



def _unbound_cache(B=2, H=4, D=64):
    """A binding Cache object whose arena is a CPU tensor and which holds no library handle:
    enough to exercise the binding's argument checks, which all run before any library call
    (a call that passed them would reach the C library with host pointers, so none does)."""
    import torch
    c = binding.Cache.__new__(binding.Cache)
    c.torch = torch
    c.B, c.H, c.D, c.L, c.G = B, H, D, 1, G
    c.arena = torch.empty(0, dtype=torch.uint8)
    c._h = None
    return c


def test_binding_rejects_wrong_tensors_before_any_call():
    import torch
    c = _unbound_cache()
    B, H, D = c.B, c.H, c.D
    f16, f32 = torch.float16, torch.float32
    q = torch.zeros(B, H, D, dtype=f16)
    cases = [
        ("wrong dtype", lambda: c.attend_draft(0, q.float())),
        ("wrong shape", lambda: c.attend_draft(0, q[:, :2].contiguous())),
        ("non-contiguous", lambda: c.attend_draft(0, torch.zeros(B, D, H, dtype=f16).transpose(1, 2))),
        ("undersized out", lambda: c.attend_draft(0, q, out=torch.empty(B, H, D - 1, dtype=f32))),
        ("out wrong dtype", lambda: c.attend_draft(0, q, out=torch.empty(B, H, D, dtype=f16))),
        ("verify q 3-d", lambda: c.attend_verify(0, q)),
        ("verify out", lambda: c.attend_verify(0, q[:, None].contiguous(),
                                               out=torch.empty(B, 2, H, D, dtype=f32))),
        ("gqa shape", lambda: c.attend_draft_gqa(0, torch.zeros(B, H * 3, D, dtype=f16), 2)),
        ("append k/v differ", lambda: c.append(0, torch.zeros(B, 3, H, D, dtype=f16),
                                                torch.zeros(B, 2, H, D, dtype=f16))),
        ("append heads", lambda: c.append(0, torch.zeros(B, 3, H + 1, D, dtype=f16),
                                           torch.zeros(B, 3, H + 1, D, dtype=f16))),
        ("counts", lambda: c.append(0, torch.zeros(B, 3, H, D, dtype=f16),
                                    torch.zeros(B, 3, H, D, dtype=f16), n=[1, 2, 3])),
        ("fused verify k", lambda: c.append_attend_verify(
            0, torch.zeros(B, 2, H, D, dtype=f16), torch.zeros(B, 2, H, D, dtype=f16),
            torch.zeros(B, 3, H, D, dtype=f16))),
        ("device out", lambda: c.attend_draft_dev(0, q, torch.empty(B, H, D + 1, dtype=f32))),
        ("not a tensor", lambda: c.attend_draft(0, q.numpy())),
    ]
    for what, call in cases:
        with pytest.raises(ValueError):
            call()
        assert c._h is None, what
