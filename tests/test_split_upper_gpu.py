"""GPU parity of the split-upper layout (qs_config.split_upper = 1: the upper nibble C_U = 4 C_T +
C_M of every code stored as a 2-bit top plane and a 2-bit middle plane) and of the top-k-bit
draft (qs_attend_draft_bits) against the CPU oracle.

The 2-bit planes, lower planes, metadata and tail must be bit-exact; attention outputs within
the parity gate.  On the same inputs, the split layout's 4-bit draft and verify must equal the
default layout's bit for bit (the same nibble values reach the same arithmetic), and a one-query
verify must equal the 2-bit draft once every code's low six bits are the draft's replacement
(C_M = 2, C_L = 0: 0b100000).
"""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import synth
from hierarchical_quantized_kv_amd.binding import Cache, QsError, QS_ERR_INVALID_ARG
from lockstep import Lockstep, log

pytestmark = pytest.mark.gpu
G = 128


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def kv(B, n, H, D, seed, outliers=None, dist="normal"):
    k, v = synth.kv_host(B, n, H, D, seed, seed + 7919, dist_k=dist, outliers=outliers)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def qd(B, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, None, H, D, seed, gain)).cuda()


def qv(B, m, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, m, H, D, seed, gain)).cuda()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("off", [8, 0])
def test_split_flush_round(D, off):
    """Group-by-group append / flush (with degenerate and all-positive groups), 2-bit and
    4-bit drafts, rollback, a 5-query verify, rollback, flush; planes bit-exact."""
    log(f"case: split upper, flush round D={D} off={off}")
    H = 3
    out = synth.outlier_channels(H, D, 1400 + D)
    ls = Lockstep(1, 1, H, D, 8 * G, 4, tag=f"split{D}o{off}", split_upper=True,
                  draft_offset=off)
    k, v = kv(1, 5 * G + 40, H, D, 1401, outliers=out)
    k, v = k.clone(), v.clone()
    k[:, :G, 0, 5] = 0.75                                    # a constant key channel
    v[:, 10:20, 0, :] = -1.5                                 # constant value rows
    k[:, 2 * G:3 * G] = k[:, 2 * G:3 * G].abs() + 2.0       # all-positive groups
    v[:, 2 * G:3 * G] = v[:, 2 * G:3 * G].abs() + 0.5
    for g in range(5):
        ls.append(0, k[:, g * G:(g + 1) * G].contiguous(), v[:, g * G:(g + 1) * G].contiguous())
        ls.flush(0)
    ls.append(0, k[:, 5 * G:].contiguous(), v[:, 5 * G:].contiguous())
    ls.check_planes(0)
    for s in range(4):
        dk, dv = kv(1, 1, H, D, 1410 + s, outliers=out)
        ls.append(0, dk, dv)
        q = qd(1, H, D, 1420 + s, gain=1.0 + s)
        ls.draft_bits(0, q, 2)
        ls.draft_bits(0, q, 4)
        ls.draft(0, q)
    ls.rollback(0, [4])
    tk, tv = kv(1, 5, H, D, 1430, outliers=out)
    ls.append(0, tk, tv)
    ls.verify(0, qv(1, 5, H, D, 1431))
    ls.rollback(0, [2])
    ls.append(0, *kv(1, 100, H, D, 1432, outliers=out))
    ls.flush(0)
    ls.check_planes(0)
    ls.draft_bits(0, qd(1, H, D, 1433, gain=4.0), 2)
    log(f"split{D}o{off}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [64, 128])
def test_split_prefill_batch_and_bitwise_match_with_the_nibble_layout(D):
    """Ragged batch prefill into a split cache and a default one from the same prompt: split
    planes bit-exact against the oracle; the split layout's 4-bit draft and verify equal the
    default layout's bit for bit; 2-bit drafts against the oracle (student-t keys)."""
    log(f"case: split upper, prefill batch D={D}")
    B, H = 3, 4
    lens = [7 * G + 45, 2 * G + 3, 90]
    ls = Lockstep(1, B, H, D, 8 * G, 6, tag=f"splitpre{D}", split_upper=True)
    plain = Cache(1, B, H, D, 8 * G, 6)
    k, v = kv(B, max(lens), H, D, 1440, dist="student_t3")
    ls.prefill(0, k, v, n=lens)
    plain.prefill(0, k, v, n=lens)
    ls.check_planes(0)
    for s in range(3):
        q = qd(B, H, D, 1441 + s, gain=2.0)
        d2 = ls.draft_bits(0, q, 2)
        d4 = ls.draft(0, q)
        assert torch.equal(d4, plain.attend_draft(0, q)), "split 4-bit draft != nibble draft"
        assert not torch.equal(d2, d4)
    m = 7
    tk, tv = kv(B, m, H, D, 1450)
    ls.append(0, tk, tv)
    plain.append(0, tk, tv)
    q = qv(B, m, H, D, 1451)
    out = ls.verify(0, q)
    assert torch.equal(out, plain.attend_verify(0, q)), "split verify != nibble verify"
    log(f"splitpre{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")
    plain.close()


@pytest.mark.parametrize("D", [64, 128])
def test_two_bit_draft_equals_one_query_verify_when_low_bits_are_its_replacement(D):
    """Every C_M set to 2 and every C_L to 0 makes each code 64 C_T + 32, the 2-bit draft's own
    reconstruction: the VALU 2-bit draft and the MFMA one-query verify (which reads all three
    planes) then agree, and each matches the oracle set up the same way."""
    log(f"case: split upper, 2-bit draft == verify(m=1), D={D}")
    H = 4
    ls = Lockstep(1, 2, H, D, 8 * G, 4, tag=f"split2dv{D}", split_upper=True)
    k, v = kv(2, 6 * G + 45, H, D, 1460)
    ls.prefill(0, k, v, n=[6 * G + 45, 3 * G + 2])
    ls.gpu.section("mk", 0).fill_(0xAA)
    ls.gpu.section("mv", 0).fill_(0xAA)
    ls.gpu.section("lk", 0).fill_(0x00)
    ls.gpu.section("lv", 0).fill_(0x00)
    ls.orc[0].set_low_bits(0, 6, 32)
    q = qd(2, H, D, 1461, gain=2.0)
    d = ls.draft_bits(0, q, 2)
    vq = ls.verify(0, q[:, None].contiguous())[:, 0]
    torch.cuda.synchronize()
    diff = float((d - vq).abs().max())
    ref = float(d.abs().max())
    log(f"split2dv{D}: max |draft2 - verify| {diff:.3e} (max |out| {ref:.3e}); vs oracle {ls.max_abs:.3e}")
    assert diff <= 5e-5 * max(ref, 1e-3)


def test_split_fused_calls_and_rejections():
    """Fused append + attend on the split layout (against append then attend, bit for bit, and
    the oracle); the calls the layout does not serve are rejected, as is a 2-bit draft on the
    default layout."""
    log("case: split upper, fused calls and rejected calls")
    H, D, B, gamma = 2, 128, 2, 4
    ls = Lockstep(1, B, H, D, 8 * G, gamma, tag="splitfused", split_upper=True)
    plain = Cache(1, B, H, D, 8 * G, gamma, split_upper=True)
    lens = [3 * G + 62, 2 * G + 10]
    k, v = kv(B, max(lens), H, D, 1470)
    ls.prefill(0, k, v, n=lens)
    plain.prefill(0, k, v, n=lens)
    kn, vn = kv(B, 1, H, D, 1471)
    q = qd(B, H, D, 1472)
    out = ls.gpu.append_attend_draft(0, kn, vn, q)
    ls.orc[0].append(0, ls._host_heads(kn, 2), ls._host_heads(vn, 2))
    ref = ls.orc[0].attend_draft(0, ls._host_heads(q, 1))
    torch.cuda.synchronize()
    ls._cmp_out(out, ref, "split fused draft")
    plain.append(0, kn, vn)
    assert torch.equal(out, plain.attend_draft(0, q))
    kt, vt = kv(B, gamma + 1, H, D, 1473)
    qm = qv(B, gamma + 1, H, D, 1474)
    out = ls.gpu.append_attend_verify(0, kt, vt, qm)
    ls.orc[0].append(0, ls._host_heads(kt, 2), ls._host_heads(vt, 2))
    ref = ls.orc[0].attend_verify(0, ls._host_heads(qm, 2))
    torch.cuda.synchronize()
    ls._cmp_out(out, ref, "split fused verify")
    plain.append(0, kt, vt)
    assert torch.equal(out, plain.attend_verify(0, qm))
    ls.check_planes(0)
    for call in (lambda: ls.gpu.attend_draft_gqa(0, qd(B, 2 * H, D, 1475), 2),
                 lambda: ls.gpu.to_device_state(),
                 lambda: ls.gpu.attend_draft_bits(0, q, 3)):
        with pytest.raises(QsError) as e:
            call()
        assert e.value.status == QS_ERR_INVALID_ARG
    nibble = Cache(1, 1, H, D, 2 * G, gamma)
    nibble.append(0, kn[:1].contiguous(), vn[:1].contiguous())
    with pytest.raises(QsError) as e:
        nibble.attend_draft_bits(0, q[:1].contiguous(), 2)
    assert e.value.status == QS_ERR_INVALID_ARG
    with pytest.raises(QsError):
        Cache(1, 1, H, D, 2 * G, gamma, split_upper=True, meta_fp16=True)
    log(f"splitfused: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")
    plain.close()
    nibble.close()
