"""GPU parity of the fp16 metadata format (qs_config.meta_fp16 = 1: per group (scale s, offset
b = -s z) in fp16, a code C standing for s C + b) against the CPU oracle in the same format.

Planes and the fp16 pairs must be bit-exact (the pairs are compared through their exact fp32
values); attention outputs within max-abs 2e-3.  Every call path of the library runs on the
format: flush, prefill, draft, verify (m up to 16), fused append + attend, grouped queries and
device mode.
"""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import synth
from hierarchical_quantized_kv_amd.binding import Cache
from lockstep import Lockstep, log

pytestmark = pytest.mark.gpu
G = 128


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def kv(B, n, H, D, seed, outliers=None):
    k, v = synth.kv_host(B, n, H, D, seed, seed + 7919, outliers=outliers)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def qd(B, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, None, H, D, seed, gain)).cuda()


def qv(B, m, H, D, seed, gain=1.0):
    return torch.from_numpy(synth.queries_host(B, m, H, D, seed, gain)).cuda()


@pytest.mark.parametrize("D", [64, 128])
def test_meta16_flush_round_and_degenerate_groups(D):
    """Append / flush group by group (one with a constant key channel, an all-zero key group,
    constant value rows, all-positive groups, a key head in the hundreds), a draft step,
    rollback, a 5-query verify, rollback, flush."""
    log(f"case: fp16 metadata, flush round D={D}")
    H = 3
    out = synth.outlier_channels(H, D, 1200 + D)
    ls = Lockstep(1, 1, H, D, 8 * G, 4, tag=f"m16flush{D}", meta_fp16=True)
    k, v = kv(1, 5 * G + 40, H, D, 1201, outliers=out)
    k, v = k.clone(), v.clone()
    k[:, :G, 0, 5] = 0.75
    k[:, G:2 * G, 1, :] = 0.0
    v[:, 10:20, 0, :] = -1.5
    k[:, 2 * G:3 * G] = k[:, 2 * G:3 * G].abs() + 2.0
    v[:, 2 * G:3 * G] = v[:, 2 * G:3 * G].abs() + 0.5
    k[:, 3 * G:4 * G, 2] = k[:, 3 * G:4 * G, 2] * 20.0 + 300.0   # offsets b ~ -220 .. -300
    for g in range(5):
        ls.append(0, k[:, g * G:(g + 1) * G].contiguous(), v[:, g * G:(g + 1) * G].contiguous())
        ls.flush(0)
    ls.append(0, k[:, 5 * G:].contiguous(), v[:, 5 * G:].contiguous())
    ls.check_planes(0)
    ls.draft(0, qd(1, H, D, 1202, gain=0.05))          # the keys of head 2 are large
    dk, dv = kv(1, 1, H, D, 1203)
    ls.append(0, dk, dv)
    ls.draft(0, qd(1, H, D, 1204, gain=0.05))
    ls.rollback(0, [1])
    tk, tv = kv(1, 5, H, D, 1205)
    ls.append(0, tk, tv)
    ls.verify(0, qv(1, 5, H, D, 1206, gain=0.05))
    ls.rollback(0, [3])
    ls.flush(0, min_tail=1)
    ls.check_planes(0)
    log(f"m16flush{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [64, 128])
def test_meta16_prefill_and_max_queries(D):
    """qs_prefill with ragged prompts (empty, G-1, a multiple of G, one after an earlier group)
    on the second layer of two, the draft constant 0, then a 16-query verify and drafts."""
    log(f"case: fp16 metadata, prefill + m=16 D={D}")
    H, B = 5, 4
    ls = Lockstep(2, B, H, D, 8 * G, 15, draft_offset=0, tag=f"m16pre{D}", meta_fp16=True)
    k0, v0 = kv(B, G, H, D, 1300)
    ls.append(1, k0, v0, [0, 0, 0, G])
    ls.flush(1)
    lens = [0, G - 1, 3 * G, 5 * G + 77]
    k, v = kv(B, max(lens), H, D, 1301 + D)
    ls.prefill(1, k, v, lens)
    ls.check_planes(1)
    k16, v16 = kv(B, 16, H, D, 1302)
    ls.append(1, k16, v16)
    ls.draft(1, qd(B, H, D, 1303), sm_scale=1.25)
    ls.verify(1, qv(B, 16, H, D, 1304), sm_scale=0.8)
    ls.rollback(1, [9, 16, 0, 3])
    ls.check_state(1)
    ls.draft(1, qd(B, H, D, 1305))
    log(f"m16pre{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("m16", [True, False])
def test_meta16_draft_equals_one_query_verify_when_lower_planes_are_the_offset(D, m16):
    """With every lower nibble set to the draft offset 8 the full code is the draft's, so the
    VALU draft and the MFMA verify (m = 1) agree, and each matches the oracle (both formats on
    the same inputs)."""
    log(f"case: fp16 metadata {m16}, draft == verify(m=1), D={D}")
    H = 4
    ls = Lockstep(1, 2, H, D, 8 * G, 4, tag=f"m16dv{D}", meta_fp16=m16)
    k, v = kv(2, 6 * G + 45, H, D, 1310)
    ls.prefill(0, k, v, n=[6 * G + 45, 3 * G + 2])
    ls.gpu.section("lk", 0).fill_(0x88)
    ls.gpu.section("lv", 0).fill_(0x88)
    ls.orc[0].set_lower_nibbles(0, 8)
    q = qd(2, H, D, 1311, gain=2.0)
    d = ls.draft(0, q)
    vq = ls.verify(0, q[:, None].contiguous())[:, 0]
    torch.cuda.synchronize()
    diff = float((d - vq).abs().max())
    ref = float(d.abs().max())
    log(f"m16dv{D} fp16={m16}: max |draft - verify| {diff:.3e} (max |out| {ref:.3e}); "
        f"vs oracle {ls.max_abs:.3e}")
    # each pass is within a few 1e-5 of the fp64 result (the draft's fixed-point weights keep
    # 22 fractional bits of the wave's largest weight; measured: up to 2.2e-5 of max |out|, all
    # of it the draft's), while a wrong nibble or offset moves the outputs by >= 1e-2
    assert diff <= 5e-5 * max(ref, 1e-3)


def test_meta16_fused_grouped_and_device_mode():
    """The other call paths on the format: fused append + attend (against append then attend,
    bit for bit, and the oracle), grouped queries (g = 4) and device-mode attention."""
    log("case: fp16 metadata, fused / grouped / device mode")
    H, D, B, gamma = 2, 128, 3, 4
    ls = Lockstep(1, B, H, D, 8 * G, 15, tag="m16paths", meta_fp16=True)
    plain = Cache(1, B, H, D, 8 * G, 15, meta_fp16=True)
    lens = [3 * G + 62, 2 * G + 10, 5 * G]
    k, v = kv(B, max(lens), H, D, 1320)
    ls.prefill(0, k, v, n=lens)
    plain.prefill(0, k, v, n=lens)
    n = [1, 2, 1]
    kn, vn = kv(B, 2, H, D, 1321)
    q = qd(B, H, D, 1322)
    out = ls.gpu.append_attend_draft(0, kn, vn, q, n=n)
    ls.orc[0].append(0, ls._host_heads(kn, 2), ls._host_heads(vn, 2), n)
    ref = ls.orc[0].attend_draft(0, ls._host_heads(q, 1))
    torch.cuda.synchronize()
    ls._cmp_out(out, ref, "m16 fused draft")
    plain.append(0, kn, vn, n)
    assert torch.equal(out, plain.attend_draft(0, q))
    kt, vt = kv(B, gamma + 1, H, D, 1323)
    qm = qv(B, gamma + 1, H, D, 1324)
    out = ls.gpu.append_attend_verify(0, kt, vt, qm)
    ls.orc[0].append(0, ls._host_heads(kt, 2), ls._host_heads(vt, 2))
    ref = ls.orc[0].attend_verify(0, ls._host_heads(qm, 2))
    torch.cuda.synchronize()
    ls._cmp_out(out, ref, "m16 fused verify")
    plain.append(0, kt, vt)
    assert torch.equal(out, plain.attend_verify(0, qm))
    ls.check_planes(0)
    # grouped queries: query head h*g + r reads cached head h
    g, mt = 4, 3
    qg = qd(B, H * g, D, 1325, gain=2.0)
    qgv = qv(B, mt, H * g, D, 1326)
    out_d = ls.gpu.attend_draft_gqa(0, qg, g)
    out_v = ls.gpu.attend_verify_gqa(0, qgv, g)
    torch.cuda.synchronize()
    for r in range(g):
        heads = [h * g + r for h in range(H)]
        ls._cmp_out(out_d[:, heads], ls.orc[0].attend_draft(0, qg[:, heads].cpu().numpy()),
                    f"m16 gqa draft r={r}")
        ls._cmp_out(out_v[:, :, heads],
                    ls.orc[0].attend_verify(0, qgv[:, :, heads].contiguous().cpu().numpy()),
                    f"m16 gqa verify r={r}")
    # device mode: the counters in the arena, the fixed plan
    od = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    ov = torch.empty((B, 3, H, D), dtype=torch.float32, device="cuda")
    qd2, qv2 = qd(B, H, D, 1327), qv(B, 3, H, D, 1328)
    ls.gpu.to_device_state()
    ls.gpu.attend_draft_dev(0, qd2, od)
    ls.gpu.attend_verify_dev(0, qv2, ov)
    assert ls.gpu.from_device_state() == 0
    torch.cuda.synchronize()
    ls._cmp_out(od, ls.orc[0].attend_draft(0, ls._host_heads(qd2, 1)), "m16 device draft")
    ls._cmp_out(ov, ls.orc[0].attend_verify(0, ls._host_heads(qv2, 2)), "m16 device verify")
    log(f"m16paths: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")
    plain.close()


def test_meta16_sections_are_half_the_fp32_ones():
    a = Cache(2, 3, 4, 128, 8 * G, 6)
    b = Cache(2, 3, 4, 128, 8 * G, 6, meta_fp16=True)
    assert b.layout.kmeta_bytes * 2 == a.layout.kmeta_bytes
    assert b.layout.vmeta_bytes * 2 == a.layout.vmeta_bytes
    assert b.section("kmeta", 1).dtype == torch.float16
    assert b.section("kmeta", 1).shape == a.section("kmeta", 1).shape
    a.close()
    b.close()
