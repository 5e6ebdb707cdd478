"""qs_spec_accept_static, the accept / correct step for callers that cannot allocate: its
workspace is the library's own device array instead of a caller buffer.  Through the C ABI it
must give exactly the results of qs_spec_accept (the same kernels over a caller workspace) on two
calls in a row, the second smaller than the first (the array keeps the first call's contents,
which the second must not read), and reject a workspace need beyond its 4 MiB.
"""
import numpy as np
import pytest
import torch

from hierarchical_quantized_kv_amd import binding
from hierarchical_quantized_kv_amd.binding import QsError, QS_ERR_BUFFER, QS_ERR_INVALID_ARG

pytestmark = pytest.mark.gpu


def _softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _case(seed, B, gamma, V):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2.0, (B, gamma + 1, V)).astype(np.float32)
    d = (t[:, :gamma] + rng.normal(0, 1.0, (B, gamma, V))).astype(np.float32)
    cdf = np.cumsum(_softmax(d), axis=-1)
    x = np.minimum((cdf < rng.random((B, gamma, 1))).sum(axis=-1), V - 1).astype(np.int32)
    u = rng.random((B, gamma + 1)).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dev(t), dev(d), dev(x), dev(u)


def _static(t, d, x, u):
    B = t.shape[0]
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    binding.spec_accept_static(t, d, x, u, n, nxt)
    return n, nxt


def test_static_workspace_matches_caller_workspace_on_two_calls():
    assert torch.cuda.is_available()
    big = (40, 6, 32000)     # workspace ~ 70 KB
    small = (3, 2, 4097)     # second call: smaller, the array still holds the first one's data
    for seed, (B, gamma, V) in ((7001, big), (7002, small)):
        print(f"case: static workspace, B={B} gamma={gamma} V={V}", flush=True)
        t, d, x, u = _case(seed, B, gamma, V)
        n_s, nxt_s = _static(t, d, x, u)
        n_r, nxt_r = binding.spec_accept(t, d, x, u)
        torch.cuda.synchronize()
        assert torch.equal(n_s, n_r) and torch.equal(nxt_s, nxt_r), (B, gamma, V)
        assert int(n_s.min()) >= 0 and int(n_s.max()) <= gamma
        assert int(nxt_s.min()) >= 0 and int(nxt_s.max()) < V


def test_static_workspace_rejects_what_does_not_fit():
    # 2048 sequences, gamma 15, a 128256-token vocabulary need ~18 MB of workspace (> 4 MiB);
    # the check comes before any launch, so small placeholder tensors are never read
    B, gamma, V = 2048, 15, 128256
    assert binding.spec_workspace_bytes(B, gamma, V) > binding.SPEC_STATIC_BYTES
    import ctypes
    one = torch.zeros(1, dtype=torch.float32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    P = ctypes.c_void_p
    st = binding.lib().qs_spec_accept_static(P(one.data_ptr()), P(one.data_ptr()),
                                             P(idx.data_ptr()), P(one.data_ptr()), B, gamma, V,
                                             P(idx.data_ptr()), P(idx.data_ptr()), None)
    assert st == QS_ERR_BUFFER
    st = binding.lib().qs_spec_accept_static(P(one.data_ptr()), P(one.data_ptr()),
                                             P(idx.data_ptr()), P(one.data_ptr()), 1, 0, 10,
                                             P(idx.data_ptr()), P(idx.data_ptr()), None)
    assert st == QS_ERR_INVALID_ARG
    # a size that fits: batch 256, gamma 15, vocab 128256 (2.2 MB)
    assert binding.spec_workspace_bytes(256, 15, 128256) <= binding.SPEC_STATIC_BYTES
