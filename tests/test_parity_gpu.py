"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Planes, metadata, tail slots and counters must be bit-exact; attention outputs must agree within
max-abs 2e-3.  Inputs are seeded synthetic fp16 tensors (see hierarchical_quantized_kv_amd.synth).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import synth
from hierarchical_quantized_kv_amd.binding import Cache
from lockstep import Lockstep, check_close, log

pytestmark = pytest.mark.gpu
G = 128


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def kv(B, n, H, D, seed, dist="normal", outliers=None):
    k, v = synth.kv_host(B, n, H, D, seed, seed + 7919, dist_k=dist, outliers=outliers)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def qd(B, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, None, H, D, seed, gain)).cuda()


def qv(B, m, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, m, H, D, seed, gain)).cuda()


def prefill(ls, layer, k, v):
    """Append + flush G tokens at a time (the 'quantize once' prompt path), remainder in tail."""
    n = k.shape[1]
    pos = 0
    while n - pos >= G:
        ls.append(layer, k[:, pos:pos + G].contiguous(), v[:, pos:pos + G].contiguous())
        ls.flush(layer)
        pos += G
    if pos < n:
        ls.append(layer, k[:, pos:].contiguous(), v[:, pos:].contiguous())


# ------------------------------------------------------------------------------------------
# Workload configurations
# ------------------------------------------------------------------------------------------

def test_config_tiny_every_op():
    """1 layer, 2 heads, D 64, ctx 1024 (8 groups) + 64-token tail; one draft step; rollback;
    verify of 5 queries; rollback of 3 rejected tokens.  Compared after every op."""
    log("case: tiny config, every op")
    H, D = 2, 64
    ls = Lockstep(1, 1, H, D, 1024 + 2 * G, 4, tag="tiny")
    k, v = kv(1, 1024 + 64, H, D, 101)
    prefill(ls, 0, k[:, :1024], v[:, :1024])
    ls.check_planes(0)
    ls.append(0, k[:, 1024:].contiguous(), v[:, 1024:].contiguous())
    ls.check_planes(0)
    dk, dv = kv(1, 1, H, D, 102)
    ls.append(0, dk, dv)
    ls.draft(0, qd(1, H, D, 103))
    ls.rollback(0, [1])
    tk, tv = kv(1, 5, H, D, 104)
    ls.append(0, tk, tv)
    ls.verify(0, qv(1, 5, H, D, 105))
    ls.rollback(0, [3])
    ls.check_planes(0)
    ls.draft(0, qd(1, H, D, 106))
    log(f"tiny: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_config_llama_layer_8k():
    """Llama-2-7B-shaped layer: 32 heads, D 128, ctx 8192, 1 % of key channels x8; one gamma=4
    speculation round."""
    log("case: llama layer 8k")
    H, D, gamma = 32, 128, 4
    out = synth.outlier_channels(H, D, synth.seed_for(2, 0, "outlier"))
    ls = Lockstep(1, 1, H, D, 8192 + 2 * G, gamma, tag="8k")
    k, v = kv(1, 8192 + 64, H, D, 201, outliers=out)
    prefill(ls, 0, k[:, :8192], v[:, :8192])
    ls.append(0, k[:, 8192:].contiguous(), v[:, 8192:].contiguous())
    ls.check_planes(0)
    for s in range(gamma):
        dk, dv = kv(1, 1, H, D, 210 + s, outliers=out)
        ls.append(0, dk, dv)
        ls.draft(0, qd(1, H, D, 220 + s))
    ls.rollback(0, [gamma])
    tk, tv = kv(1, gamma + 1, H, D, 230, outliers=out)
    ls.append(0, tk, tv)
    ls.verify(0, qv(1, gamma + 1, H, D, 231))
    ls.rollback(0, [gamma - 2])
    ls.flush(0)
    ls.check_planes(0)
    log(f"8k: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


# ------------------------------------------------------------------------------------------
# Edge cases
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("nt", [1, 63, 64, 65, 200, 256])
def test_tail_only(D, nt):
    log(f"case: tail only D={D} nt={nt}")
    H = 3
    ls = Lockstep(1, 1, H, D, 2 * G, 15, tag=f"tail{D}/{nt}")
    k, v = kv(1, nt, H, D, 300 + nt)
    ls.append(0, k, v)
    ls.draft(0, qd(1, H, D, 301), sm_scale=0.9)
    for m in sorted({1, min(nt, 7), min(nt, 16)}):
        ls.verify(0, qv(1, m, H, D, 302 + m), sm_scale=1.1)


@pytest.mark.parametrize("D", [64, 128])
def test_quantized_only_and_ring_wrap(D):
    log(f"case: quantized only / ring wrap D={D}")
    H = 4
    ls = Lockstep(1, 1, H, D, 6 * G, 6, tag=f"qonly{D}")
    k, v = kv(1, 5 * G + 100, H, D, 400)
    prefill(ls, 0, k[:, :3 * G], v[:, :3 * G])       # nt = 0, head = G
    ls.draft(0, qd(1, H, D, 401))
    ls.append(0, k[:, 3 * G:4 * G + 100].contiguous(), v[:, 3 * G:4 * G + 100].contiguous())
    ls.flush(0)                                       # head back to 0, 100 left in the tail
    ls.append(0, k[:, 4 * G + 100:].contiguous(), v[:, 4 * G + 100:].contiguous())
    ls.check_planes(0)
    ls.draft(0, qd(1, H, D, 402))
    ls.verify(0, qv(1, 7, H, D, 403))


def test_ragged_batch_and_many_chunks():
    """Sequences with different quantized/tail lengths in one call; 260 groups x 32 heads forces
    multi-group chunks with a short last chunk."""
    log("case: ragged batch, many chunks")
    H, D, B = 32, 128, 3
    ls = Lockstep(1, B, H, D, 264 * G, 4, heads=[0, 17, 31], tag="ragged")
    lens = [260 * G + 37, 3 * G + 9, 90]
    n_max = max(lens)
    k, v = kv(B, n_max, H, D, 500)
    pos = 0
    while pos < n_max:
        n = [max(0, min(G, L - pos)) for L in lens]
        ls.append(0, k[:, pos:pos + G].contiguous(), v[:, pos:pos + G].contiguous(), n)
        ls.flush(0)
        pos += G
    ls.check_planes(0)
    ls.draft(0, qd(B, H, D, 501))
    ls.verify(0, qv(B, 5, H, D, 502))
    ls.rollback(0, [3, 4, 2])
    ls.draft(0, qd(B, H, D, 503))


@pytest.mark.parametrize("B", [1, 2, 8, 9, 64])
def test_batch_buckets(B):
    """The kernels are instantiated for batches of 1, up to 8 and up to 64 sequences; each size
    here lands on a bucket edge.  Ragged lengths: tail-only, quantized-only and mixed sequences."""
    log(f"case: batch bucket B={B}")
    H, D = 2, 64
    ls = Lockstep(1, B, H, D, 6 * G, 4, tag=f"bucket{B}")
    lens = [(97 * b + 61) % (5 * G) + 1 for b in range(B)]
    lens[-1] = 4 * G
    n_max = max(lens)
    k, v = kv(B, n_max, H, D, 700 + B)
    pos = 0
    while pos < n_max:
        n = [max(0, min(G, L - pos)) for L in lens]
        ls.append(0, k[:, pos:pos + G].contiguous(), v[:, pos:pos + G].contiguous(), n)
        if pos + G <= n_max:
            ls.flush(0)
        pos += G
    ls.check_planes(0)
    ls.draft(0, qd(B, H, D, 701 + B))
    k5, v5 = kv(B, 5, H, D, 704 + B)
    ls.append(0, k5, v5)
    ls.verify(0, qv(B, 5, H, D, 702 + B))
    ls.rollback(0, [b % 5 for b in range(B)])
    ls.check_state(0)
    ls.draft(0, qd(B, H, D, 703 + B))


@pytest.mark.parametrize("D", [64, 128])
def test_max_queries_offset0_odd_heads(D):
    """The largest verify (m = 16 queries, gamma_max 15), the draft constant off = 0, scales other
    than 1, an odd head count (uneven XCD shares) and the second layer of a two-layer cache."""
    log(f"case: m=16, off=0, 5 heads, D={D}")
    H, B = 5, 2
    ls = Lockstep(2, B, H, D, 8 * G, 15, draft_offset=0, tag=f"m16_{D}")
    k, v = kv(B, 5 * G + 40, H, D, 800 + D)
    prefill(ls, 1, k, v)
    ls.check_planes(1)
    ls.draft(1, qd(B, H, D, 801), sm_scale=1.25)
    k16, v16 = kv(B, 16, H, D, 802 + D)
    ls.append(1, k16, v16)
    ls.verify(1, qv(B, 16, H, D, 803), sm_scale=0.8)
    ls.rollback(1, [9, 16])
    ls.check_state(1)
    ls.draft(1, qd(B, H, D, 804), sm_scale=0.8)
    log(f"m16_{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_matches_quantize_once(D):
    """qs_prefill (whole groups quantized straight from the prompt, the rest to the tail) against
    the oracle's quantize-once prefill: ragged prompts (empty, G-1, an exact multiple, and one
    after an earlier group), then round verbs on top."""
    log(f"case: prefill D={D}")
    H, B = 4, 4
    ls = Lockstep(1, B, H, D, 8 * G, 6, tag=f"prefill{D}")
    k0, v0 = kv(B, G, H, D, 900)
    ls.append(0, k0, v0, [0, 0, 0, G])
    ls.flush(0)
    lens = [0, G - 1, 3 * G, 5 * G + 77]
    k, v = kv(B, max(lens), H, D, 901 + D)
    ls.prefill(0, k, v, lens)
    ls.check_planes(0)
    k1, v1 = kv(B, 7, H, D, 902)
    ls.append(0, k1, v1)
    ls.draft(0, qd(B, H, D, 903))
    ls.verify(0, qv(B, 7, H, D, 904))
    ls.rollback(0, [3, 3, 3, 3])
    ls.flush(0)
    ls.check_planes(0)
    log(f"prefill{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_prefill_of_whole_groups_only():
    """Prompts that are whole groups (no rest row in the launch), an empty prompt (no launch at
    all), then a prompt with a rest on top of the first: planes, tail and counters against the
    oracle."""
    log("case: prefill of whole groups only")
    H, B, D = 3, 2, 128
    ls = Lockstep(1, B, H, D, 8 * G, 4, tag="prefillwhole")
    k, v = kv(B, 2 * G, H, D, 950)
    ls.prefill(0, k, v, [2 * G, G])
    ls.check_planes(0)
    nq, nt, _ = ls.check_state(0)
    assert list(nq) == [2 * G, G] and list(nt) == [0, 0]
    ls.prefill(0, k, v, [0, 0])
    ls.check_state(0)
    k2, v2 = kv(B, G + 9, H, D, 951)
    ls.prefill(0, k2, v2, [G + 9, 5])
    ls.check_planes(0)
    nq, nt, _ = ls.check_state(0)
    assert list(nq) == [3 * G, G] and list(nt) == [9, 5]
    ls.draft(0, qd(B, H, D, 952))
    log(f"prefillwhole: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_degenerate_groups():
    """Constant key channels and value rows (scale clamped to 1e-8, huge zero-point) and
    all-positive groups (zero-point below 0)."""
    log("case: degenerate groups")
    H, D = 2, 128
    ls = Lockstep(1, 1, H, D, 4 * G, 4, tag="degenerate")
    k, v = kv(1, 3 * G + 20, H, D, 600)
    k, v = k.clone(), v.clone()
    k[:, :G, 0, 5] = 0.75           # constant key channel in group 0
    k[:, G:2 * G, 1, :] = 0.0       # all-zero key group
    v[:, 10:20, 0, :] = -1.5        # constant value rows
    k[:, 2 * G:3 * G] = k[:, 2 * G:3 * G].abs() + 2.0   # all-positive keys in group 2
    v[:, 2 * G:3 * G] = v[:, 2 * G:3 * G].abs() + 0.5
    prefill(ls, 0, k, v)
    ls.check_planes(0)
    ls.draft(0, qd(1, H, D, 601))
    ls.verify(0, qv(1, 5, H, D, 602))


@pytest.mark.parametrize("gain", [4.0, 8.0])
def test_peaky_softmax(gain):
    log(f"case: peaky softmax gain={gain}")
    H, D = 4, 128
    ls = Lockstep(1, 1, H, D, 8 * G, 6, tag=f"peaky{gain}")
    out = synth.outlier_channels(H, D, 700)
    k, v = kv(1, 7 * G + 30, H, D, 701, outliers=out)
    prefill(ls, 0, k, v)
    ls.draft(0, qd(1, H, D, 702, gain))
    ls.verify(0, qv(1, 7, H, D, 703, gain))
    log(f"peaky{gain}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [64, 128])
def test_draft_equals_one_query_verify_when_lower_planes_are_the_offset(D):
    """With every lower nibble of the arena set to the draft offset 8, the full code is the draft
    reconstruction, so a one-query verify equals the draft: two independent GPU paths (signed
    4-bit integer dot products; MFMA over 1024 + C8) agree, and each matches the oracle with the
    same nibbles."""
    log(f"case: draft == verify(m=1) with lower planes 8, D={D}")
    H = 4
    ls = Lockstep(1, 2, H, D, 8 * G, 4, tag=f"dv{D}")
    k, v = kv(2, 6 * G + 45, H, D, 910)
    ls.prefill(0, k, v, n=[6 * G + 45, 3 * G + 2])
    ls.gpu.section("lk", 0).fill_(0x88)
    ls.gpu.section("lv", 0).fill_(0x88)
    ls.orc[0].set_lower_nibbles(0, 8)
    q = qd(2, H, D, 911, gain=2.0)
    d = ls.draft(0, q)
    vq = ls.verify(0, q[:, None].contiguous())[:, 0]
    torch.cuda.synchronize()
    diff = float((d - vq).abs().max())
    ref = float(d.abs().max())
    log(f"dv{D}: max |draft - verify| {diff:.3e} (max |out| {ref:.3e}); vs oracle {ls.max_abs:.3e}")
    # each pass is within a few 1e-5 of the fp64 result (the draft's fixed-point weights keep
    # 22 fractional bits of the wave's largest weight; measured: up to 2.2e-5 of max |out|, all
    # of it the draft's), while a wrong nibble or offset moves the outputs by >= 1e-2
    assert diff <= 5e-5 * max(ref, 1e-3)


@pytest.mark.parametrize("D,B", [(64, 3), (128, 3), (64, 9)])
def test_fused_append_attend_equals_append_then_attend(D, B):
    """qs_append_attend_draft / _verify give the oracle's outputs and, bit for bit, the outputs,
    ring contents and counters of qs_append followed by qs_attend_*: ragged per-sequence counts,
    new tokens straddling a 64-token tail chunk, a sequence whose ring head is G, and a fused
    verify after the draft tokens are rolled back."""
    log(f"case: fused append + attend D={D} B={B}")
    H, gamma = 4, 4
    ls = Lockstep(1, B, H, D, 8 * G, gamma, tag=f"fused{D}x{B}")
    plain = Cache(1, B, H, D, 8 * G, gamma)
    base = [3 * G + 62, 2 * G + 10, 5 * G]              # heads G, 0, G; tails 62, 10, 0
    lens = [base[b % 3] + 5 * (b // 3) for b in range(B)]
    k, v = kv(B, max(lens), H, D, 940 + B)
    ls.prefill(0, k, v, n=lens)
    plain.prefill(0, k, v, n=lens)
    # per-step counts, by sequence mod 3; the second step crosses 64 in sequence 0
    step_n = [[row[b % 3] for b in range(B)]
              for row in ([1, 1, 1], [2, 0, 1], [1, 2, 0], [1, 1, 1])]
    for i, n in enumerate(step_n):
        kn, vn = kv(B, max(n), H, D, 950 + i)
        q = qd(B, H, D, 960 + i)
        out = ls.gpu.append_attend_draft(0, kn, vn, q, n=n)
        ls.orc[0].append(0, ls._host_heads(kn, 2), ls._host_heads(vn, 2), n)
        ref = ls.orc[0].attend_draft(0, ls._host_heads(q, 1))
        torch.cuda.synchronize()
        ls._cmp_out(out, ref, f"fused draft {i}")
        plain.append(0, kn, vn, n)
        assert torch.equal(out, plain.attend_draft(0, q)), i
    drop = [[2, 2, 1][b % 3] for b in range(B)]
    ls.rollback(0, drop)
    plain.rollback(0, drop)
    kv_, vv_ = kv(B, gamma + 1, H, D, 970)
    qm = qv(B, gamma + 1, H, D, 971)
    out = ls.gpu.append_attend_verify(0, kv_, vv_, qm)
    ls.orc[0].append(0, ls._host_heads(kv_, 2), ls._host_heads(vv_, 2))
    ref = ls.orc[0].attend_verify(0, ls._host_heads(qm, 2))
    torch.cuda.synchronize()
    ls._cmp_out(out, ref, "fused verify")
    plain.append(0, kv_, vv_)
    assert torch.equal(out, plain.attend_verify(0, qm))
    ls.check_planes(0)                                   # ring slots bit-exact vs the oracle
    assert all(np.array_equal(x, y) for x, y in zip(ls.gpu.state(0), plain.state(0)))
    nq, nt, head = plain.state(0)
    for b in range(B):
        slots = [(int(head[b]) + j) % (2 * G) for j in range(int(nt[b]))]
        for name in ("tail_k", "tail_v"):
            assert torch.equal(ls.gpu.section(name, 0)[b][:, slots].view(torch.int16),
                               plain.section(name, 0)[b][:, slots].view(torch.int16)), (b, name)
    assert head.tolist() == [[G, 0, G][b % 3] for b in range(B)]
    plain.close()


def test_grouped_verify_in_two_calls_matches_one_causal_verify():
    """A grouped verify wider than one call's query columns (7 tokens x 4 query heads = 28 >
    gamma_max + 1) run as two append + verify calls (4 tokens, then 3): each call's tokens see the
    tail causally, so together they equal the oracle's single 7-token verify of every query head
    (per r, over the cached heads)."""
    log("case: grouped verify of 7 tokens x 4 query heads in two calls")
    H, D, g, m = 2, 128, 4, 7
    ls = Lockstep(1, 1, H, D, 8 * G, 15, tag="gqa-split")
    k, v = kv(1, 3 * G + 50, H, D, 1201)
    ls.prefill(0, k, v)
    kt, vt = kv(1, m, H, D, 1202)
    q = qv(1, m, H * g, D, 1203)
    ls.gpu.append(0, kt[:, :4].contiguous(), vt[:, :4].contiguous())
    out1 = ls.gpu.attend_verify_gqa(0, q[:, :4].contiguous(), g)
    ls.gpu.append(0, kt[:, 4:].contiguous(), vt[:, 4:].contiguous())
    out2 = ls.gpu.attend_verify_gqa(0, q[:, 4:].contiguous(), g)
    torch.cuda.synchronize()
    ls.orc[0].append(0, kt.cpu().numpy(), vt.cpu().numpy())
    for r in range(g):
        heads = [h * g + r for h in range(H)]
        ref = ls.orc[0].attend_verify(0, q[:, :, heads].contiguous().cpu().numpy())
        ls._cmp_out(out1[:, :, heads], ref[:, :4], f"split verify first r={r}")
        ls._cmp_out(out2[:, :, heads], ref[:, 4:], f"split verify second r={r}")
    log(f"gqa split verify: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D,g,mt,B", [(128, 4, 4, 3), (64, 2, 3, 3), (128, 8, 1, 3),
                                      (64, 16, 1, 3), (128, 4, 2, 1), (64, 3, 5, 1),
                                      (64, 8, 2, 2), (128, 9, 1, 2)])
def test_grouped_queries_match_the_oracle(D, g, mt, B):
    """Grouped queries: query head h*g + r attends over cached head h.  The reference is the
    oracle's own draft / verify over the cached heads, called once per r with the queries of
    heads h*g + r.  Ragged batch: a tail-only sequence, one with a two-chunk tail.  The drafts
    with g <= 8 run the paired MFMA form (g = 8: all 16 columns), g = 9 and 16 the 16-column
    form."""
    log(f"case: grouped queries D={D} g={g} m={mt} B={B}")
    H = 2
    ls = Lockstep(1, B, H, D, 8 * G, 15, tag=f"gqa{D}x{g}x{mt}x{B}")
    lens = [5 * G + 70, 100, 3 * G][:B]
    k, v = kv(B, max(lens), H, D, 980 + g)
    ls.prefill(0, k, v, n=lens)
    kt, vt = kv(B, mt, H, D, 985 + g + B)
    ls.append(0, kt, vt)                                 # the verified tokens are tail tokens
    qd_ = qd(B, H * g, D, 990 + g, gain=2.0)
    qv_ = qv(B, mt, H * g, D, 991 + g)
    out_d = ls.gpu.attend_draft_gqa(0, qd_, g)
    out_v = ls.gpu.attend_verify_gqa(0, qv_, g)
    torch.cuda.synchronize()
    for r in range(g):
        heads = [h * g + r for h in range(H)]
        ref_d = ls.orc[0].attend_draft(0, qd_[:, heads].cpu().numpy())
        ref_v = ls.orc[0].attend_verify(0, qv_[:, :, heads].contiguous().cpu().numpy())
        ls._cmp_out(out_d[:, heads], ref_d, f"gqa draft r={r}")
        ls._cmp_out(out_v[:, :, heads], ref_v, f"gqa verify r={r}")
    if g == 8:  # one query head per cached head through the grouped path: the plain draft
        q1 = qd(B, H, D, 995)
        d1 = ls.gpu.attend_draft_gqa(0, q1, 1)
        d0 = ls.gpu.attend_draft(0, q1)
        torch.cuda.synchronize()
        diff = float((d1 - d0).abs().max())
        log(f"gqa g=1 MFMA draft vs VALU draft: max abs diff {diff:.2e}")
        assert diff <= 2e-5
    log(f"gqa{D}x{g}x{mt}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_result_does_not_depend_on_the_split():
    """The split-K log-sum-exp merge reaches one softmax whatever the split: one sequence's
    outputs alone (many workers per head), inside a batch of 8 (few workers per head), and in
    device mode (a fixed plan) agree to 2e-6 of their size (measured: up to 7e-7)."""
    log("case: split invariance")
    H, D, n = 32, 128, 40 * G + 77
    k, v = kv(1, n, H, D, 920)
    q = qd(1, H, D, 921)
    qm = qv(1, 5, H, D, 922)
    solo = Cache(1, 1, H, D, 48 * G, 4)
    solo.prefill(0, k, v)
    batch = Cache(1, 8, H, D, 48 * G, 4)
    lens = [n if b == 5 else (b * 7 + 3) * G // 2 + 11 * b + 5 for b in range(8)]
    assert all(L % G >= 5 for L in lens)           # the 5-query verify needs nt >= 5
    kb, vb = kv(8, n, H, D, 930)
    kb[5], vb[5] = k[0], v[0]
    batch.prefill(0, kb, vb, n=lens)
    qb, qmb = qd(8, H, D, 931), qv(8, 5, H, D, 932)
    qb[5], qmb[5] = q[0], qm[0]
    outs = {"solo": (solo.attend_draft(0, q)[0], solo.attend_verify(0, qm)[0]),
            "batch": (batch.attend_draft(0, qb)[5], batch.attend_verify(0, qmb)[5])}
    od = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
    ov = torch.empty((1, 5, H, D), dtype=torch.float32, device="cuda")
    solo.to_device_state()
    solo.attend_draft_dev(0, q, od)
    solo.attend_verify_dev(0, qm, ov)
    assert solo.from_device_state() == 0
    outs["device"] = (od[0], ov[0])
    torch.cuda.synchronize()
    for name in ("batch", "device"):
        for i, what in enumerate(("draft", "verify")):
            a, b = outs["solo"][i], outs[name][i]
            rel = float((a - b).abs().max()) / float(a.abs().max())
            log(f"split: {what} solo vs {name}: max rel diff {rel:.2e}")
            assert rel <= 2e-6, (what, name, rel)
    solo.close()
    batch.close()


def test_grid_exact_cache_verify_equals_fp16_attention():
    """Keys/values on the quantization grid: the verify pass must equal plain fp16 attention
    (torch float64 on the CPU) -- a check of the GPU path that does not go through the oracle."""
    log("case: grid-exact cache")
    rng = np.random.default_rng(800)
    H, D, ng = 2, 128, 4
    n = ng * G
    kk = rng.integers(0, 256, size=(n, H, D))
    for g in range(ng):
        kk[g * G] = 0
        kk[g * G + 1] = 255
    kz = np.repeat(rng.integers(0, 256, size=(ng, H, D)), G, axis=0)
    vk = rng.integers(0, 256, size=(n, H, D))
    vk[:, :, 0], vk[:, :, 1] = 0, 255
    vz = rng.integers(0, 256, size=(n, H, 1))
    kx = ((kk - kz) * 2.0 ** -5).astype(np.float16)[None]
    vx = ((vk - vz) * 2.0 ** -5).astype(np.float16)[None]
    ls = Lockstep(1, 1, H, D, ng * G, 4, tag="grid")
    tk, tv = kv(1, 30, H, D, 801)
    prefill(ls, 0, torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda())
    ls.append(0, tk, tv)
    q = qv(1, 5, H, D, 802)
    out = ls.verify(0, q).cpu().numpy()
    kall = np.concatenate([kx[0], tk[0].cpu().numpy()]).astype(np.float64)
    vall = np.concatenate([vx[0], tv[0].cpu().numpy()]).astype(np.float64)
    qq = q[0].cpu().numpy().astype(np.float64)
    N = kall.shape[0]
    for h in range(H):
        s = qq[:, h] @ kall[:, h].T
        for i in range(5):
            s[i, N - 5 + i + 1:] = -np.inf
        p = np.exp(s - s.max(1, keepdims=True))
        ref = (p @ vall[:, h]) / p.sum(1, keepdims=True)
        check_close(out[0, :, h], ref, f"grid head {h}")


def test_errors_leave_state_unchanged_on_gpu():
    log("case: error paths")
    from hierarchical_quantized_kv_amd.binding import Cache, QsError, QS_ERR_CAPACITY, QS_ERR_STATE
    H, D = 2, 64
    c = Cache(1, 2, H, D, G, 4)
    k, v = kv(2, 2 * G + 1, H, D, 900)
    with pytest.raises(QsError) as e:
        c.append(0, k, v)
    assert e.value.status == QS_ERR_CAPACITY
    c.append(0, k[:, :10].contiguous(), v[:, :10].contiguous(), [10, 3])
    with pytest.raises(QsError) as e:
        c.rollback(0, [1, 4])
    assert e.value.status == QS_ERR_STATE
    with pytest.raises(QsError) as e:
        c.attend_verify(0, qv(2, 4, H, D, 901))
    assert e.value.status == QS_ERR_STATE
    nq, nt, hd = c.state(0)
    assert list(nt) == [10, 3] and list(nq) == [0, 0]


@pytest.mark.parametrize("D", [64, 128])
def test_draft_over_many_calls(D):
    """60 consecutive drafts -- plain and fused with the token's append, a ragged batch whose
    work plans change as the contexts grow and flush (a tail-only sequence among them) -- each
    against the oracle; then a device-mode draft (its own plan and kernels) on the same state
    agrees within 1e-5 of max |out|."""
    log(f"case: draft, 60 calls, D={D}")
    B, H = 3, 4
    ls = Lockstep(1, B, H, D, 24 * G, 6, tag=f"calls{D}")
    lens = [9 * G + 17, 2 * G + 100, 30]
    k, v = kv(B, max(lens), H, D, 1500 + D)
    ls.prefill(0, k, v, n=lens)
    for call in range(60):
        kn, vn = kv(B, 1, H, D, 1600 + call)
        q = qd(B, H, D, 1700 + call, gain=1.0 + (call % 5))
        if call % 2:
            out = ls.gpu.append_attend_draft(0, kn, vn, q)
            ls.orc[0].append(0, ls._host_heads(kn, 2), ls._host_heads(vn, 2))
            ref = ls.orc[0].attend_draft(0, ls._host_heads(q, 1))
            torch.cuda.synchronize()
            ls._cmp_out(out, ref, f"fused draft {call}")
        else:
            ls.append(0, kn, vn)
            ls.draft(0, q)
        if call % 10 == 9:
            big_k, big_v = kv(B, G, H, D, 1800 + call)
            ls.append(0, big_k, big_v, n=[G, G // 2, 3])
            ls.flush(0)
    q = qd(B, H, D, 1900)
    host = ls.draft(0, q)
    od = torch.empty_like(host)
    ls.gpu.to_device_state()
    ls.gpu.attend_draft_dev(0, q, od)
    assert ls.gpu.from_device_state() == 0
    torch.cuda.synchronize()
    diff = float((host - od).abs().max())
    ref = float(host.abs().max())
    log(f"calls{D}: 60 calls, max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}; "
        f"host vs device mode {diff:.2e} of {ref:.2e}")
    assert diff <= 1e-5 * ref
