"""The parity gate (tests/parity_gate.py) can fail at full size: CPU-only checks with the oracle.

At 128k context the draft / verify outputs are a few 1e-3 in size, so the absolute bound of
2e-3 alone would accept a kernel that skipped or double-counted one of the 1024 quantized
groups of a head.  These tests build such a wrong result with the oracle itself (the cache of
the same token stream with one group removed, or with one group present twice) and check that
the absolute bound is indeed blind to it while the per-row relative bound rejects it.
"""
import numpy as np
import pytest

import oracle
from oracle import OracleCache
from hierarchical_quantized_kv_amd import synth
from parity_gate import ATOL, RTOL_ROW, check_close, compare

G = 128


def setup_module(_):
    oracle.build(force=False)


def _outputs(k, v, tail, groups, q, qv, H, D):
    """Draft and verify outputs of an oracle cache holding `groups` (indices into the groups of
    k / v, in that order) followed by the fp16 tail tokens."""
    kk = np.concatenate([k[:, g * G:(g + 1) * G] for g in groups], axis=1)
    vv = np.concatenate([v[:, g * G:(g + 1) * G] for g in groups], axis=1)
    orc = OracleCache(1, 1, H, D, G, (len(groups) + 1) * G, 6)
    orc.prefill(0, kk, vv)
    orc.append(0, tail[0], tail[1])
    return orc.attend_draft(0, q), orc.attend_verify(0, qv)


@pytest.mark.parametrize("wrong", ["dropped", "doubled"])
def test_row_gate_catches_one_group_of_1024(wrong):
    H, D, ng = 2, 128, 1024  # 131072 quantized tokens per head
    out = synth.outlier_channels(H, D, 77)
    k, v = synth.kv_host(1, ng * G + 64, H, D, 71, 72, outliers=out)
    tail = (k[:, ng * G:], v[:, ng * G:])
    q = synth.queries_host(1, None, H, D, 73)
    qv = synth.queries_host(1, 7, H, D, 74)
    ref_d, ref_v = _outputs(k, v, tail, list(range(ng)), q, qv, H, D)
    j = 517
    groups = [g for g in range(ng) if g != j] if wrong == "dropped" else \
        list(range(j + 1)) + list(range(j, ng))
    got_d, got_v = _outputs(k, v, tail, groups, q, qv, H, D)
    for got, ref, what in ((got_d, ref_d, "draft"), (got_v, ref_v, "verify")):
        mad, rel = compare(got, ref)
        print(f"{wrong} group, {what}: max abs {mad:.2e} (bound {ATOL}), worst row rel {rel:.2e}")
        assert rel > 10 * RTOL_ROW
        with pytest.raises(AssertionError):
            check_close(got, ref, what)
        if what == "draft":  # the draft's outputs are small enough that 2e-3 alone is blind
            assert mad <= ATOL


def test_gate_accepts_rounding_level_differences():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((1, 7, 4, 128)) * 3e-3
    got = ref * (1 + 1e-5 * rng.standard_normal(ref.shape))
    mad, rel = check_close(got, ref, "rounding")
    assert rel < 1e-4 and mad < 1e-6


def test_gate_rejects_non_finite_and_shape_mismatch():
    ref = np.ones((2, 64))
    got = ref.copy()
    got[1, 3] = np.nan
    with pytest.raises(AssertionError):
        check_close(got, ref, "nan")
    with pytest.raises(AssertionError):
        check_close(np.ones((2, 32)), ref, "shape")
