"""GPU parity at the full sizes of the workloads (the launch configurations the benchmark times),
checked on sampled heads / layers that the CPU oracle can afford.

  * LWM-128k-shaped layer: 32 heads x 128, 131072 prefilled tokens, gamma = 6 round, with plain
    queries and with queries x8 (a peaky softmax); the same prefilled layer in both metadata
    formats.
  * head_dim 64: the same round on a 128k layer of 32 heads x 64 channels.
  * Grouped queries: a Llama-3.1-8B-shaped 128k layer (8 cached heads x 4 query heads), the
    grouped draft (plain and x8 queries) and a 4-token grouped verify on sampled cached heads.
  * Device mode: a gamma = 6 round and a flush through the device-mode verbs on a 128k layer.
  * LWM-128k-shaped layer in the split-upper layout: the 2-bit draft (plain and x8 queries),
    the 4-bit draft and verify over one prefilled layer.
  * LWM-128k-shaped stack: all 32 layers of the 128k cache the benchmark times (4 x 8 GiB of
    planes), every layer prefilled; a gamma = 6 round on every layer checked on layers 0 and 31
    (sampled heads), then an all-layer flush and the planes of both layers bit-exact.
  * Llama-2-7B-32K-shaped stack: 32 layers, 32768 tokens, 64 rounds of gamma = 4 with
    Bernoulli(0.9) acceptance driving rollback and flush; outputs checked every 8th round on
    three layers, final planes of every layer checked bit-exact against the oracle's replay.
  * Batched stress: 8 sequences with ragged lengths in [16384, 32768], Student-t(3) keys,
    gamma = 4 with per-sequence acceptance until each sequence has 512 generated tokens.

Inputs are generated on the GPU (torch's seeded generator) and the sampled heads are copied to
the host for the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import synth
from lockstep import Lockstep, log

pytestmark = pytest.mark.gpu
G = 128


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def dev_kv(config, layer, B, n, H, D, dist="normal", outliers=None, salt=0):
    return synth.kv_device(torch, B, n, H, D, synth.seed_for(config, layer, "k") + 7 * salt,
                           synth.seed_for(config, layer, "v") + 7 * salt, "cuda", dist_k=dist,
                           outliers=outliers)


def dev_q(shape, gen, D):
    return (torch.randn(shape, generator=gen, device="cuda") / math.sqrt(D)).to(torch.float16)


def prefill(ls, layer, k, v, lens=None):
    n = k.shape[1]
    pos = 0
    while pos < n:
        kk, vv = k[:, pos:pos + G].contiguous(), v[:, pos:pos + G].contiguous()
        cnt = None if lens is None else [max(0, min(G, L - pos)) for L in lens]
        ls.append(layer, kk, vv, cnt)
        ls.flush(layer)
        pos += G


def test_lwm_128k_layer():
    log("case: LWM-128k layer, heads 0/13/31 sampled")
    H, D, ctx, gamma = 32, 128, 131072, 6
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, gamma, heads=[0, 13, 31], tag="128k")
    out = synth.outlier_channels(H, D, synth.seed_for(4, 0, "outlier"))
    k, v = dev_kv(4, 0, 1, ctx + 64, H, D, outliers=out)
    prefill(ls, 0, k[:, :ctx], v[:, :ctx])
    ls.append(0, k[:, ctx:].contiguous(), v[:, ctx:].contiguous())
    del k, v
    gen = torch.Generator(device="cuda").manual_seed(4000)
    for s in range(gamma):
        dk, dv = dev_kv(4, 0, 1, 1, H, D, outliers=out, salt=s + 1)
        ls.append(0, dk, dv)
        ls.draft(0, dev_q((1, H, D), gen, D))
    # a peaky softmax: the same cache, queries x8
    ls.draft(0, (dev_q((1, H, D), gen, D).float() * 8).half())
    ls.rollback(0, [gamma])
    tk, tv = dev_kv(4, 0, 1, gamma + 1, H, D, outliers=out, salt=100)
    ls.append(0, tk, tv)
    ls.verify(0, dev_q((1, gamma + 1, H, D), gen, D))
    ls.verify(0, (dev_q((1, gamma + 1, H, D), gen, D).float() * 8).half())
    ls.rollback(0, [3])
    ls.flush(0)
    ls.check_planes(0)
    log(f"128k: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_head_dim_64_128k_layer():
    """The same round on a 128k layer of 32 heads x 64 channels (the head_dim-64 instantiations
    at full size: two lanes per key row in the draft, the verify's half-width tiles)."""
    log("case: head_dim 64, 128k layer, heads 0/17/31 sampled")
    H, D, ctx, gamma = 32, 64, 131072, 6
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, gamma, heads=[0, 17, 31], tag="128k-d64")
    out = synth.outlier_channels(H, D, synth.seed_for(4, 1, "outlier"))
    k, v = dev_kv(4, 1, 1, ctx + 64, H, D, outliers=out)
    prefill(ls, 0, k[:, :ctx], v[:, :ctx])
    ls.append(0, k[:, ctx:].contiguous(), v[:, ctx:].contiguous())
    del k, v
    gen = torch.Generator(device="cuda").manual_seed(4064)
    for s in range(gamma):
        dk, dv = dev_kv(4, 1, 1, 1, H, D, outliers=out, salt=s + 1)
        ls.append(0, dk, dv)
        ls.draft(0, dev_q((1, H, D), gen, D))
    ls.draft(0, (dev_q((1, H, D), gen, D).float() * 8).half())
    ls.rollback(0, [gamma])
    tk, tv = dev_kv(4, 1, 1, gamma + 1, H, D, outliers=out, salt=100)
    ls.append(0, tk, tv)
    ls.verify(0, dev_q((1, gamma + 1, H, D), gen, D))
    ls.rollback(0, [3])
    ls.flush(0)
    ls.check_planes(0)
    log(f"128k d64: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("D", [128, 64])
def test_grouped_queries_128k_layer(D):
    """Grouped queries at the size the benchmark times: a Llama-3.1-8B-shaped layer of 8 cached
    heads shared by 4 query heads each, head_dim 128 (and the same at head_dim 64, whose paired
    draft runs at 4 waves per SIMD), 131072 prefilled tokens plus a tail, the
    grouped draft (32 query heads, plain and x8) and a 4-token grouped verify (16 query columns
    per cached head), checked on cached heads 0, 5 and 7 against the oracle's passes over those
    heads."""
    log(f"case: grouped queries, 128k layer, head_dim {D}, 8 cached heads x 4, cached heads "
        f"0/5/7 sampled")
    H, ctx, g, mt = 8, 131072, 4, 4
    sampled = [0, 5, 7]
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, 15, heads=sampled, tag=f"gqa128k-d{D}")
    out = synth.outlier_channels(H, D, synth.seed_for(4, 2, "outlier"))
    k, v = dev_kv(4, 2, 1, ctx + 64 + mt, H, D, outliers=out)
    ls.prefill(0, k[:, :ctx + 64].contiguous(), v[:, :ctx + 64].contiguous())
    ls.append(0, k[:, ctx + 64:].contiguous(), v[:, ctx + 64:].contiguous())
    del k, v
    gen = torch.Generator(device="cuda").manual_seed(4128)
    qd_ = dev_q((1, H * g, D), gen, D)
    qd8 = (dev_q((1, H * g, D), gen, D).float() * 8).half()   # a peaky softmax
    qv_ = dev_q((1, mt, H * g, D), gen, D)
    out_d = ls.gpu.attend_draft_gqa(0, qd_, g)
    out_d8 = ls.gpu.attend_draft_gqa(0, qd8, g)
    out_v = ls.gpu.attend_verify_gqa(0, qv_, g)
    torch.cuda.synchronize()
    for r in range(g):
        heads = [h * g + r for h in sampled]
        ref_d = ls.orc[0].attend_draft(0, qd_[:, heads].cpu().numpy())
        ref_d8 = ls.orc[0].attend_draft(0, qd8[:, heads].cpu().numpy())
        ref_v = ls.orc[0].attend_verify(0, qv_[:, :, heads].contiguous().cpu().numpy())
        ls._cmp_out(out_d[:, heads], ref_d, f"gqa draft r={r}")
        ls._cmp_out(out_d8[:, heads], ref_d8, f"gqa draft x8 r={r}")
        ls._cmp_out(out_v[:, :, heads], ref_v, f"gqa verify r={r}")
    log(f"gqa 128k d{D}: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_device_mode_128k_layer():
    """Device mode at full size: the fixed work plan of the device-mode verbs (workers dealt
    groups w, w + W, .. of whatever the sequence holds) over a 128k layer, one gamma = 6 round
    of appends, drafts, rollback and verify, then an all-layer flush, against the oracle on
    heads 0 and 31, and the counters and planes once back in host mode."""
    log("case: device mode, 128k layer, heads 0/31 sampled")
    H, D, ctx, gamma = 32, 128, 131072, 6
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, gamma, heads=[0, 31], tag="dev128k")
    out = synth.outlier_channels(H, D, synth.seed_for(4, 3, "outlier"))
    k, v = dev_kv(4, 3, 1, ctx + 64, H, D, outliers=out)
    ls.prefill(0, k, v)
    del k, v
    ls.gpu.to_device_state()
    gen = torch.Generator(device="cuda").manual_seed(4200)
    od = torch.empty((1, H, D), dtype=torch.float32, device="cuda")
    for s in range(gamma):
        dk, dv = dev_kv(4, 3, 1, 1, H, D, outliers=out, salt=s + 1)
        q = dev_q((1, H, D), gen, D)
        ls.gpu.append_dev(0, dk, dv)
        ls.gpu.attend_draft_dev(0, q, od)
        ls.orc[0].append(0, ls._host_heads(dk, 2), ls._host_heads(dv, 2))
        ref = ls.orc[0].attend_draft(0, ls._host_heads(q, 1))
        torch.cuda.synchronize()
        ls._cmp_out(od[:, ls.heads], ref, f"dev draft {s}")
    tk, tv = dev_kv(4, 3, 1, gamma + 1, H, D, outliers=out, salt=100)
    qv_ = dev_q((1, gamma + 1, H, D), gen, D)
    ov = torch.empty((1, gamma + 1, H, D), dtype=torch.float32, device="cuda")
    ls.gpu.rollback_dev(0, gamma)
    ls.gpu.append_dev(0, tk, tv)
    ls.gpu.attend_verify_dev(0, qv_, ov)
    ls.orc[0].rollback(0, [gamma])
    ls.orc[0].append(0, ls._host_heads(tk, 2), ls._host_heads(tv, 2))
    ref = ls.orc[0].attend_verify(0, ls._host_heads(qv_, 2))
    torch.cuda.synchronize()
    ls._cmp_out(ov[:, :, ls.heads], ref, "dev verify")
    ls.gpu.rollback_dev(0, 3)
    ls.orc[0].rollback(0, [3])
    ls.gpu.flush_dev(-1, G)
    ls.orc[0].flush(0, G)
    assert ls.gpu.from_device_state() == 0
    ls.check_planes(0)
    log(f"dev 128k: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_lwm_128k_32_layer_stack():
    """The full 32-layer 128k arena: every layer prefilled, a gamma = 6 round on all layers
    (outputs of layers 0 and 31 against the oracle on sampled heads), 64 more tokens so that
    the all-layer flush quantizes a group of every layer at the far end of each plane section,
    then the live planes, metadata and tail of layers 0 and 31 bit-exact."""
    L, H, D, ctx, gamma = 32, 32, 128, 131072, 6
    log("case: LWM-128k 32-layer stack, layers 0/31, heads 0/19/31 sampled")
    ls = Lockstep(L, 1, H, D, ctx + 4 * G, gamma, heads=[0, 19, 31], layers=[0, L - 1],
                  tag="128kx32")
    outs = [synth.outlier_channels(H, D, synth.seed_for(4, l, "outlier")) for l in range(L)]
    for l in range(L):
        k, v = dev_kv(4, l, 1, ctx + 64, H, D, outliers=outs[l])
        ls.prefill(l, k, v)
        del k, v
    torch.cuda.synchronize()
    log("128kx32: prefill of 32 layers done")
    gen = torch.Generator(device="cuda").manual_seed(4200)
    for s in range(gamma):
        for l in range(L):
            dk, dv = dev_kv(4, l, 1, 1, H, D, outliers=outs[l], salt=300 + s)
            ls.append(l, dk, dv)
            q = dev_q((1, H, D), gen, D)
            if s == gamma - 1:
                q = (q.float() * 8).half()  # the last draft step with a peaky softmax
            ls.draft(l, q) if l in ls.orc else ls.gpu.attend_draft(l, q)
    ls.rollback(-1, [gamma])
    for l in range(L):
        tk, tv = dev_kv(4, l, 1, gamma + 1, H, D, outliers=outs[l], salt=400)
        ls.append(l, tk, tv)
        q = dev_q((1, gamma + 1, H, D), gen, D)
        ls.verify(l, q) if l in ls.orc else ls.gpu.attend_verify(l, q)
    ls.rollback(-1, [2])
    for l in range(L):
        tk, tv = dev_kv(4, l, 1, 64, H, D, outliers=outs[l], salt=500)
        ls.append(l, tk, tv)
    ls.flush(-1)
    for l in ls.layers:
        nq, nt, _ = ls.check_state(l)
        assert int(nq[0]) == ctx + G and int(nt[0]) == 64 + (gamma + 1 - 2) + 64 - G
        ls.check_planes(l)
    ls.draft(L - 1, dev_q((1, H, D), gen, D))
    log(f"128kx32: layers 0/31 bit-exact after the all-layer flush; max abs {ls.max_abs:.3e} "
        f"max rel {ls.max_rel:.3e}")


def test_lwm_128k_split_upper_layer():
    """A 128k layer in the split-upper layout (top and middle 2-bit planes): one qs_prefill of
    131072 + 64 tokens, the 2-bit draft (qs_attend_draft_bits) with plain queries and with
    queries x8, the 4-bit draft and a 7-query verify over the same planes, all against the
    oracle on sampled heads (the 2-bit draft's weights are on five digits: this checks their
    rounding over a whole 128k context), then the planes bit-exact."""
    log("case: LWM-128k layer, split-upper layout, heads 0/17/31 sampled")
    H, D, ctx, gamma = 32, 128, 131072, 6
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, gamma, heads=[0, 17, 31], tag="128ksplit",
                  split_upper=True)
    out = synth.outlier_channels(H, D, synth.seed_for(4, 2, "outlier"))
    k, v = dev_kv(4, 2, 1, ctx + 64, H, D, outliers=out)
    ls.prefill(0, k, v)
    del k, v
    ls.check_planes(0)
    gen = torch.Generator(device="cuda").manual_seed(4300)
    for s in range(2):
        dk, dv = dev_kv(4, 2, 1, 1, H, D, outliers=out, salt=600 + s)
        ls.append(0, dk, dv)
        q = dev_q((1, H, D), gen, D)
        ls.draft_bits(0, q, 2)
        ls.draft_bits(0, (q.float() * 8).half(), 2)
        ls.draft(0, q)
    tk, tv = dev_kv(4, 2, 1, gamma + 1, H, D, outliers=out, salt=700)
    ls.append(0, tk, tv)
    ls.verify(0, dev_q((1, gamma + 1, H, D), gen, D))
    log(f"128ksplit: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


@pytest.mark.parametrize("meta_fp16", [False, True])
def test_prefill_128k_layer(meta_fp16):
    """One qs_prefill of a 131072 + 64-token prompt (1024 groups quantized straight from the
    prompt, 64 tokens to the tail), bit-exact against the oracle on sampled heads, then one
    round of attention on top; in both metadata formats."""
    log(f"case: 128k prefill, heads 0/17/31 sampled, fp16 metadata {meta_fp16}")
    H, D, ctx, gamma = 32, 128, 131072, 6
    ls = Lockstep(1, 1, H, D, ctx + 4 * G, gamma, heads=[0, 17, 31], tag="prefill128k",
                  meta_fp16=meta_fp16)
    out = synth.outlier_channels(H, D, synth.seed_for(4, 1, "outlier"))
    k, v = dev_kv(4, 1, 1, ctx + 64, H, D, outliers=out)
    ls.prefill(0, k, v)
    del k, v
    ls.check_planes(0)
    gen = torch.Generator(device="cuda").manual_seed(4100)
    ls.draft(0, dev_q((1, H, D), gen, D))
    tk, tv = dev_kv(4, 1, 1, gamma + 1, H, D, outliers=out, salt=200)
    ls.append(0, tk, tv)
    ls.verify(0, dev_q((1, gamma + 1, H, D), gen, D))
    log(f"prefill128k: max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")


def test_llama_32k_full_stack_64_rounds():
    L, H, D, ctx, gamma = 32, 32, 128, 32768, 4
    log("case: 32k full stack, 64 rounds")
    check_layers = [0, 17, 31]
    ls = Lockstep(L, 1, H, D, ctx + 4 * G, gamma, heads=[0, 31], tag="32k")
    outs = [synth.outlier_channels(H, D, synth.seed_for(3, l, "outlier")) for l in range(L)]
    for l in range(L):
        k, v = dev_kv(3, l, 1, ctx + 64, H, D, outliers=outs[l])
        prefill(ls, l, k, v)
    torch.cuda.synchronize()
    log("32k: prefill done")
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(3, 0, "accept")))
    gen = torch.Generator(device="cuda").manual_seed(3000)
    for rnd in range(64):
        check = rnd % 8 == 7
        for s in range(gamma):
            for l in range(L):
                dk, dv = dev_kv(3, l, 1, 1, H, D, outliers=outs[l], salt=1000 + 10 * rnd + s)
                ls.append(l, dk, dv)
                q = dev_q((1, H, D), gen, D)
                if check and l in check_layers:
                    ls.draft(l, q)
                else:
                    ls.gpu.attend_draft(l, q)
        a = synth.acceptance(rng, gamma)
        for l in range(L):
            ls.rollback(l, [gamma])
            tk, tv = dev_kv(3, l, 1, gamma + 1, H, D, outliers=outs[l], salt=5000 + rnd)
            ls.append(l, tk, tv)
            q = dev_q((1, gamma + 1, H, D), gen, D)
            if check and l in check_layers:
                ls.verify(l, q)
            else:
                ls.gpu.attend_verify(l, q)
            ls.rollback(l, [gamma - a])
        ls.flush(-1)
        if check:
            log(f"32k: round {rnd} checked, max abs {ls.max_abs:.3e}")
    for l in range(L):
        ls.check_planes(l)
    log(f"32k: planes of all {L} layers bit-exact; max abs {ls.max_abs:.3e} rel {ls.max_rel:.3e}")


def test_batched_ragged_student_t():
    B, H, D, gamma = 8, 32, 128, 4
    log("case: batched ragged stress")
    lens = [int(x) for x in synth.ragged_lengths(B, 16384, 32768, synth.seed_for(5, 0, "len"))]
    ls = Lockstep(1, B, H, D, 32768 + 8 * G, gamma, heads=[0, 31], tag="batch8")
    k, v = dev_kv(5, 0, B, max(lens), H, D, dist="student_t3")
    prefill(ls, 0, k, v, lens)
    del k, v
    nq, nt, _ = ls.check_state(0)
    log(f"batch8: prefilled {list(nq + nt)}")
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(5, 0, "accept")))
    gen = torch.Generator(device="cuda").manual_seed(5000)
    generated = np.zeros(B, dtype=np.int64)
    rnd = 0
    while generated.min() < 512:
        check = rnd % 16 == 0
        for s in range(gamma):
            dk, dv = dev_kv(5, 0, B, 1, H, D, dist="student_t3", salt=1000 + 10 * rnd + s)
            ls.append(0, dk, dv)
            q = dev_q((B, H, D), gen, D)
            ls.draft(0, q) if check else ls.gpu.attend_draft(0, q)
        ls.rollback(0, [gamma] * B)
        tk, tv = dev_kv(5, 0, B, gamma + 1, H, D, dist="student_t3", salt=9000 + rnd)
        ls.append(0, tk, tv)
        q = dev_q((B, gamma + 1, H, D), gen, D)
        ls.verify(0, q) if check else ls.gpu.attend_verify(0, q)
        acc = np.array([synth.acceptance(rng, gamma) for _ in range(B)])
        ls.rollback(0, list(gamma - acc))
        generated += acc + 1
        ls.flush(0)
        rnd += 1
    ls.check_planes(0)
    q = dev_q((B, H, D), gen, D)
    ls.draft(0, q)
    log(f"batch8: {rnd} rounds, max abs {ls.max_abs:.3e} rel {ls.max_rel:.3e}")
