"""Benchmark of the decode-attention hot path of the hierarchical INT8 KV cache on one GPU.

Workload (default): LWM-128k-shaped cache, 32 layers x 32 heads x head_dim 128, batch 1, 131072
prefilled tokens (1024 quantized groups per head) plus a 64-token fp16 tail, keys with 1 % of
channels scaled x8.  One step is one speculation round over all layers:
  gamma = 6 draft steps (per layer: append 1 token, draft attention),
  per layer: rollback gamma, append gamma+1 target tokens, verify attention (7 queries),
  acceptance a ~ Bernoulli(0.9) until first reject, rollback gamma - a, then one flush call.
Inputs are seeded synthetic fp16 tensors resident in HBM before timing starts.  HIP events time
each timed step's run of draft calls and its run of verify calls (a call's time is its share of
the run).  After the timed steps, a bulk flush (one G-token half of every layer and head in one
launch) is timed on its own.

Prints one JSON line: value = algorithmic HBM bytes of the step / step time (GB/s), with the
roofline of the draft kernel (and of verify and flush), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step and HBM GB/s (draft & verify) at 32k/128k ctx"
PEAK_HBM_GBS = 8000.0
CPU_SAMPLE_HEADS = 16   # heads of layer 0 in the CPU-oracle sample, at least


def host_cpus():
    """(CPUs this process may run on, CPUs the OS reports)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return aff, os.cpu_count() or aff


def cpu_sample_heads(threads, H):
    """Heads in the oracle sample: at least CPU_SAMPLE_HEADS, and one per thread (up to H)."""
    return max(1, min(H, max(CPU_SAMPLE_HEADS, threads)))
G = 128
# device sources of the cache's kernels (the traffic figures are tied to their hash)
KERNEL_SRCS = [os.path.join(ROOT, "hierarchical_quantized_kv_amd", "csrc", f) for f in (
    "qs_args.h", "qs_device.h", "qs_attn_host.hip", "qs_attn_app.hip", "qs_attn_dev.hip",
    "qs_attn_gqa.hip", "qs_attn_split_host.hip", "qs_attn_split_app.hip", "qs_quant.hip")]
PROFILES = os.path.join(ROOT, "profiles")
# HBM byte counters of rocprofv3, scaled by what they read for a plain device copy of known size
# (FETCH_SIZE counts half of the bytes a copy kernel reads; WRITE_SIZE counts them all).
# (Batch 1: the kernels' batch-bucket template argument is 1.)
# Kernel names (as rocprofv3 prints them) of the default step: the attention kernels of the
# fused append + attend calls (mode 2); --no-fuse runs the mode-0 ones.
# The attention kernels' last three arguments: the metadata format (false: fp32 (scale,
# zero-point)), the upper-plane layout (0: one 4-bit plane) and the paired MFMA form (used by the
# grouped-query draft only).
KERNELS = {"draft": "attn_kernel<128, true, 1, 2, false, 0, false>",
           "verify": "attn_kernel<128, false, 1, 2, false, 0, false>",
           "combine": "combine_kernel<128, 1, 2, 0>", "flush": "flush_kernel<128>",
           "prefill": "prefill_kernel<128>"}


def kernel_names(fuse):
    mode = 2 if fuse else 0
    return (f"attn_kernel<128, true, 1, {mode}, false, 0, false>",
            f"attn_kernel<128, false, 1, {mode}, false, 0, false>",
            f"combine_kernel<128, 1, {mode}, 0>")

CONFIGS = {
    3: dict(name="Llama-2-7B-32K-shaped full stack", layers=32, heads=32, D=128, ctx=32768,
            gamma=4),
    4: dict(name="LWM-128k-shaped", layers=32, heads=32, D=128, ctx=131072, gamma=6),
}


def draft_bytes(nq, nt, H, D, mb=8, bits=4):
    """Algorithmic bytes of one draft call: the key/value bits the draft reads (the upper
    nibble planes, or the top 2-bit planes for bits = 2) + (s, z) metadata (mb bytes a pair: 8
    fp32, 4 fp16) of every quantized token-head, the fp16 tail, the query and the fp32
    output."""
    per_tok = 2 * (D * bits // 8) + mb * D // G + mb
    return H * (nq * per_tok + nt * 4 * D + 2 * D + 4 * D)


def verify_bytes(nq, nt, H, D, m, mb=8):
    per_tok = D + D + mb * D // G + mb
    return H * (nq * per_tok + nt * 4 * D + m * (2 * D + 4 * D))


def flush_bytes(H, D):
    """One flushed G-token half per head: fp16 keys and values read, both planes of both
    written, key (s, z) per channel and value (s, z) per token written."""
    return H * (G * D * 2 * 2 + 2 * G * D + 8 * D + 8 * G)


def append_bytes(n, H, D):
    return 2 * n * H * D * 2 * 2


def prefill_bytes(n, H, D):
    """One layer's prompt of n tokens: flush bytes for each whole group, append bytes for the
    rest."""
    return (n // G) * flush_bytes(H, D) + append_bytes(n % G, H, D)


def time_steps(torch, cache, stream, dev, config, L, H, D, gamma, steps, warmup, fuse):
    """Runs `warmup` untimed and `steps` timed speculation rounds over all L layers of `cache`
    (each: gamma x (append 1 + draft) per layer, rollback gamma, append gamma+1 + verify,
    rollback by the rejected count, flush), inputs resident in HBM.  In each timed step, one
    pair of HIP events brackets the step's gamma x L draft calls and one pair its L verify calls
    (with fused calls nothing else runs on the GPU between them; a rollback is host bookkeeping),
    so a call's time is its share of the run of calls as the step executes them: events around
    single calls add their own marker cost (measured: ~6 us per call at 32k, where the step's
    128 draft and 32 verify calls at those per-call times would add up to more than the whole
    step)."""
    from hierarchical_quantized_kv_amd import synth
    m = gamma + 1
    n_steps = warmup + steps
    gen = torch.Generator(device=dev).manual_seed(12345)
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(config, 0, "accept")))
    accept = [synth.acceptance(rng, gamma) for _ in range(n_steps)]

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=gen, device=dev) * scale).to(torch.float16)

    steps_in = []
    for s in range(n_steps):
        steps_in.append(dict(
            dk=rnd(gamma, L, 1, 1, H, D), dv=rnd(gamma, L, 1, 1, H, D),
            qd=rnd(gamma, L, 1, H, D, scale=1 / math.sqrt(D)),
            tk=rnd(L, 1, m, H, D), tv=rnd(L, 1, m, H, D),
            qv=rnd(L, 1, m, H, D, scale=1 / math.sqrt(D))))
    out_d = torch.empty((1, H, D), dtype=torch.float32, device=dev)
    out_v = torch.empty((1, m, H, D), dtype=torch.float32, device=dev)
    ev = {"draft": [], "verify": []}

    def events(timed):
        if not timed:
            return None, None
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        return e0, e1

    def run_step(s, timed):
        x = steps_in[s]
        nbytes = 0
        # A draft step is the token's append followed by the draft call; fused (the default)
        # both are one call, whose bytes then include the append (without fusion the bracketed
        # run also holds the append kernels).
        e0, e1 = events(timed)
        call_bytes = 0
        for j in range(gamma):
            for layer in range(L):
                if not fuse:
                    cache.append(layer, x["dk"][j, layer], x["dv"][j, layer])
                nq, nt, _ = cache.state(layer)
                nt_call = int(nt[0]) + (1 if fuse else 0)
                db = draft_bytes(int(nq[0]), nt_call, H, D)
                nbytes += append_bytes(1, H, D) + db
                call_bytes += db + (append_bytes(1, H, D) if fuse else 0)
                if fuse:
                    cache.append_attend_draft(layer, x["dk"][j, layer], x["dv"][j, layer],
                                              x["qd"][j, layer], out=out_d)
                else:
                    cache.attend_draft(layer, x["qd"][j, layer], out=out_d)
        if timed:
            e1.record(stream)
            ev["draft"].append((e0, e1, call_bytes, gamma * L))
        e0, e1 = events(timed)
        call_bytes = 0
        for layer in range(L):
            cache.rollback(layer, [gamma])
            if not fuse:
                cache.append(layer, x["tk"][layer], x["tv"][layer])
            nq, nt, _ = cache.state(layer)
            vb = verify_bytes(int(nq[0]), int(nt[0]) + (m if fuse else 0), H, D, m)
            nbytes += append_bytes(m, H, D) + vb
            call_bytes += vb + (append_bytes(m, H, D) if fuse else 0)
            if fuse:
                cache.append_attend_verify(layer, x["tk"][layer], x["tv"][layer], x["qv"][layer],
                                           out=out_v)
            else:
                cache.attend_verify(layer, x["qv"][layer], out=out_v)
            cache.rollback(layer, [gamma - accept[s]])
        if timed:
            e1.record(stream)
            ev["verify"].append((e0, e1, call_bytes, L))
        flushed = cache.flush(-1)
        nbytes += int(flushed[0]) * L * flush_bytes(H, D)
        return nbytes

    for s in range(warmup):
        run_step(s, False)
    torch.cuda.synchronize()
    step_bytes = []
    t0 = time.perf_counter()
    for s in range(warmup, n_steps):
        step_bytes.append(run_step(s, True))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    total_bytes = sum(step_bytes)
    return dict(ms_per_step=elapsed * 1e3 / steps, value=total_bytes / elapsed / 1e9,
                elapsed=elapsed, total_bytes=total_bytes, ev=ev, steps_in=steps_in,
                accept=accept, out_d=out_d, out_v=out_v, gen=gen)


def summarize_events(events):
    """(us per call, GB/s, bytes per call, samples dropped) of (event, event, bytes, calls)
    samples, each a run of consecutive calls.  A sample whose time per call is above twice the
    median is left out, and counted (an interval can hold a stall of the host thread)."""
    t = np.array([a.elapsed_time(b) * 1e3 for a, b, _, _ in events])   # us
    by = np.array([n for _, _, n, _ in events], dtype=np.float64)
    calls = np.array([c for _, _, _, c in events], dtype=np.float64)
    per = t / calls
    keep = per <= 2.0 * np.median(per)
    avg_us = float(t[keep].sum() / calls[keep].sum())
    bytes_per_call = float(by[keep].sum() / calls[keep].sum())
    return avg_us, bytes_per_call / (avg_us * 1e-6) / 1e9, bytes_per_call, int((~keep).sum())


def measure_ctx32k(torch, stream, dev, steps, warmup, fuse):
    """The Llama-2-7B-32K-shaped stack (32 layers x 32 heads x head_dim 128, ctx 32768 + 64-token
    tail, gamma 4) run with the same step as the headline workload on a cache of its own:
    step time, and the draft / verify calls' times (events, as for the headline)."""
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache
    cfg = CONFIGS[3]
    L, H, D, ctx, gamma = cfg["layers"], cfg["heads"], cfg["D"], cfg["ctx"], cfg["gamma"]
    cache = Cache(L, 1, H, D, ctx + 16 * G, gamma)
    for layer in range(L):
        out_ch = synth.outlier_channels(H, D, synth.seed_for(3, layer, "outlier"))
        k, v = synth.kv_device(torch, 1, ctx + 64, H, D, synth.seed_for(3, layer, "k"),
                               synth.seed_for(3, layer, "v"), dev, outliers=out_ch)
        cache.prefill(layer, k, v)
        del k, v
    torch.cuda.synchronize()
    st = time_steps(torch, cache, stream, dev, 3, L, H, D, gamma, steps, warmup, fuse)
    d_us, d_gbs, d_bytes, d_drop = summarize_events(st["ev"]["draft"])
    v_us, v_gbs, v_bytes, v_drop = summarize_events(st["ev"]["verify"])
    ms_per_step, value = st["ms_per_step"], st["value"]
    cache.close()
    del cache, st
    torch.cuda.empty_cache()
    return {"workload": f"{cfg['name']}: {L} layers x {H} heads x head_dim {D}, batch 1, ctx "
                        f"{ctx} + 64-token tail, gamma {gamma} ({gamma + 1}-query verify), 1% key "
                        f"channels x8; fused append + attend calls",
            "ms_per_step": round(ms_per_step, 4), "value_gbs": round(value, 2),
            "draft_us": round(d_us, 2), "draft_bytes": int(d_bytes), "draft_gbs": round(d_gbs, 1),
            "draft_frac": round(d_gbs / PEAK_HBM_GBS, 4),
            "verify_us": round(v_us, 2), "verify_bytes": int(v_bytes),
            "verify_gbs": round(v_gbs, 1), "verify_frac": round(v_gbs / PEAK_HBM_GBS, 4),
            "samples_dropped": {"draft": d_drop, "verify": v_drop}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=4, choices=sorted(CONFIGS))
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fuse", action="store_true",
                    help="separate append and attention calls instead of the fused ones")
    ap.add_argument("--no-gqa", action="store_true",
                    help="skip the grouped-query layer (gqa: null)")
    ap.add_argument("--no-meta16", action="store_true",
                    help="skip the fp16-metadata comparison (meta16: null)")
    ap.add_argument("--no-ctx32k", action="store_true",
                    help="skip the 32k stack's step (ctx32k: null; implied by --config 3)")
    ap.add_argument("--no-topk", action="store_true",
                    help="skip the top-k-bit draft comparison (topk: null)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed step (graph_step: null)")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="host threads of the second, all-cores oracle timing (default: the "
                         "CPUs this process may run on)")
    ap.add_argument("--flush-reps", type=int, default=20,
                    help="timed all-layer flushes (each quantizes one G-token half per head)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this size first (reference "
                         "kernel for scaling HBM byte counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic profile from two rocprofv3 --pmc output folders "
                         "(FETCH_SIZE, WRITE_SIZE) of this script and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        write_traffic_summary(*args.traffic_summary, args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache

    cfg = CONFIGS[args.config]
    L = args.layers or cfg["layers"]
    H, D, ctx, gamma = cfg["heads"], cfg["D"], cfg["ctx"], cfg["gamma"]
    m = gamma + 1
    cpu_threads = args.cpu_threads or host_cpus()[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    max_ctx = ctx + 32 * G  # room for the steps' flushes and the timed bulk flushes
    print(f"bench: config {args.config} ({cfg['name']}), {L} layers, ctx {ctx}", file=sys.stderr,
          flush=True)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 19  # fp16 elements
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    # Short launches (a layer's prefill, the bulk flush) are timed behind a spin kernel of
    # ~200 us: otherwise the GPU can sit idle when it reaches the first event and the interval
    # would include the host's launch latency of the timed call.
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1_000_000)
    c1.record(stream)
    torch.cuda.synchronize()
    spin_cycles = int(1_000_000 * 200.0 / max(c0.elapsed_time(c1) * 1e3, 1.0))

    # Prefill ("quantize once"): each layer's ctx + 64-token prompt in one qs_prefill call (ctx / G
    # groups quantized, 64 tokens to the tail), timed in runs of four layers' calls.
    cache = Cache(L, 1, H, D, max_ctx, gamma)
    t0 = time.time()
    cpu_inputs = None
    pf_ev = []
    PF_RUN = 4  # layers prefilled back to back between one pair of events
    for l0 in range(0, L, PF_RUN):
        run = []
        for layer in range(l0, min(L, l0 + PF_RUN)):
            out_ch = synth.outlier_channels(H, D, synth.seed_for(args.config, layer, "outlier"))
            run.append((layer,) + synth.kv_device(torch, 1, ctx + 64, H, D,
                                                  synth.seed_for(args.config, layer, "k"),
                                                  synth.seed_for(args.config, layer, "v"), dev,
                                                  outliers=out_ch))
        torch.cuda._sleep(spin_cycles)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for layer, k, v in run:
            cache.prefill(layer, k, v)
        e1.record(stream)
        pf_ev.append((e0, e1, len(run) * prefill_bytes(ctx + 64, H, D), len(run)))
        if l0 == 0 and not args.no_cpu_baseline:
            hs = list(range(cpu_sample_heads(cpu_threads, H)))
            k, v = run[0][1], run[0][2]
            cpu_inputs = (k[:, :, hs].cpu().numpy(), v[:, :, hs].cpu().numpy())
        del run
    torch.cuda.synchronize()
    print(f"bench: prefill done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    fuse = not args.no_fuse
    st = time_steps(torch, cache, stream, dev, args.config, L, H, D, gamma, args.steps,
                    args.warmup, fuse)
    steps_in, accept, out_d, out_v, ev = st["steps_in"], st["accept"], st["out_d"], st["out_v"], st["ev"]
    ms_per_step, value, elapsed = st["ms_per_step"], st["value"], st["elapsed"]
    total_bytes = st["total_bytes"]
    print(f"bench: {args.steps} timed steps in {elapsed:.3f}s", file=sys.stderr, flush=True)
    gen = st["gen"]

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=gen, device=dev) * scale).to(torch.float16)

    # The same step replayed from a HIP graph (device mode): the step's calls are captured once
    # with the counters in device memory, and each replay advances them on the device; only the
    # step's accepted count is copied into a device word before each replay.  Bytes per step
    # from a host mirror of the counters (every layer sees the same calls).
    graph_line = None if args.no_graph else measure_graph_steps(
        torch, cache, steps_in[0], accept, args, L, H, D, gamma, m, out_d, out_v, dev, stream)

    # Bulk flush (outside the timed steps): each qs_flush(-1) quantizes one G-token half of
    # every (layer, head) in a single launch.  Every layer's tail is emptied (rolled back) and
    # refilled with 2G tokens, then two flushes run back to back between one pair of events,
    # behind the spin kernel (like the prefill): a call's time is half the pair's, so one
    # launch's marker and dispatch latency is shared by two calls, as calls queued behind other
    # work share it in a round.
    fk, fv = rnd(1, 2 * G, H, D), rnd(1, 2 * G, H, D)
    fl_ev = []
    for _ in range((args.flush_reps + 1) // 2):
        for layer in range(L):
            _, nt_l, _ = cache.state(layer)
            cache.rollback(layer, [int(nt_l[0])])
            cache.append(layer, fk, fv)
        torch.cuda._sleep(spin_cycles)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f1 = cache.flush(-1)
        f2 = cache.flush(-1)
        e1.record(stream)
        assert int(f1[0]) == 1 and int(f2[0]) == 1
        fl_ev.append((e0, e1, 2 * L * flush_bytes(H, D), 2))
    torch.cuda.synchronize()

    # The accept / correct step after verify (qs_spec_accept): synthetic fp32 logits over a
    # 32000-token vocabulary, gamma drafted tokens, fresh uniforms per call; for one sequence (the
    # workload's batch) and for 32 (where the step is bound by reading the logits).  Algorithmic
    # bytes: every logit read once; the kernels read them once for the row statistics, the one
    # or two rows of each sequence's rejection point again, and one 4096-token part of those a
    # third time.
    from hierarchical_quantized_kv_amd.binding import spec_accept, spec_workspace_bytes
    V_SPEC = 32000
    sa_ev = {1: [], 32: []}
    for sb in sa_ev:
        sa_t = torch.randn((sb, gamma + 1, V_SPEC), generator=gen, device=dev) * 2
        sa_d = sa_t[:, :gamma] + torch.randn((sb, gamma, V_SPEC), generator=gen, device=dev)
        sa_x = torch.randint(0, V_SPEC, (sb, gamma), generator=gen, device=dev, dtype=torch.int32)
        sa_ws = torch.empty(spec_workspace_bytes(sb, gamma, V_SPEC), dtype=torch.uint8, device=dev)
        for _ in range(8):
            sa_u = torch.rand((sb, gamma + 1), generator=gen, device=dev)
            torch.cuda._sleep(spin_cycles)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            spec_accept(sa_t, sa_d, sa_x, sa_u, workspace=sa_ws, stream=stream)
            e1.record(stream)
            sa_ev[sb].append((e0, e1, sb * (2 * gamma + 1) * V_SPEC * 4, 1))
        torch.cuda.synchronize()
        del sa_t, sa_d
    torch.cuda.synchronize()

    # Average over the sampled calls.  An event interval can also hold a stall of the host
    # thread; samples above twice the median (per call) are left out, and the count of those is
    # reported.
    dropped = {}

    def summarize(events, kind):
        us, gbs, nbytes, n_drop = summarize_events(events)
        dropped[kind] = n_drop
        return us, gbs, nbytes

    d_us, d_gbs, d_bytes = summarize(ev["draft"], "draft")
    v_us, v_gbs, v_bytes = summarize(ev["verify"], "verify")
    f_us, f_gbs, f_bytes = summarize(fl_ev, "flush")
    p_us, p_gbs, p_bytes = summarize(pf_ev, "prefill")
    sa = {sb: summarize(e, f"spec_accept_batch{sb}") for sb, e in sa_ev.items()}

    ctx32k = None if (args.no_ctx32k or args.config == 3) else measure_ctx32k(
        torch, stream, dev, args.steps, args.warmup, fuse)
    gqa = None if args.no_gqa else measure_gqa(torch, stream, spin_cycles, dev)
    meta16 = None if args.no_meta16 else measure_meta16(
        torch, stream, spin_cycles, dev, cfg["name"], ctx=cfg["ctx"], H=cfg["heads"],
        m=cfg["gamma"] + 1)
    topk = None if args.no_topk else measure_topk(
        torch, stream, spin_cycles, dev, cfg["name"], ctx=cfg["ctx"], H=cfg["heads"],
        m=cfg["gamma"] + 1)
    read_ceiling = measure_read_ceiling(torch, stream, {"draft": d_bytes, "verify": v_bytes})
    mixed_ceiling = measure_mixed_ceiling(torch, stream)

    cpu = None
    cpu_all = None
    if cpu_inputs is not None:
        cpu = cpu_baseline(cpu_inputs, ctx, D, gamma, threads=1)
        cpu_all = cpu_baseline(cpu_inputs, ctx, D, gamma, threads=cpu_threads)

    traffic = load_traffic(args.config)

    kn = kernel_names(fuse)

    def roof(kind, gbs, nbytes, us, kernel, launches=1):
        t = traffic.get(kind) if traffic else None
        return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": None if t is None else int(round(t * launches)),
                "bytes_per_launch": int(nbytes), "avg_launch_us": round(us, 2)}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: {L} layers x {H} heads x head_dim {D}, batch 1, "
                               f"ctx {ctx} + 64-token tail, gamma {gamma} ({m}-query verify), "
                               f"1% key channels x8",
                   "layers": L, "heads": H, "head_dim": D, "ctx": ctx, "gamma": gamma,
                   "batch": 1, "group": G, "fused_append": fuse,
                   "metadata": "fp32 (scale, zero-point)"},
        "draft_us_per_layer": round(d_us, 2),
        "draft_gbs": round(d_gbs, 1),
        "verify_us_per_layer": round(v_us, 2),
        "verify_gbs": round(v_gbs, 1),
        "flush_us_all_layers": round(f_us, 2),
        "flush_gbs": round(f_gbs, 1),
        "prefill_us_per_layer": round(p_us, 2),
        "prefill_gbs": round(p_gbs, 1),
        "roofline": roof("draft", d_gbs, d_bytes, d_us,
                         f"draft call{' (fused append)' if fuse else ''}: {kn[0]} + {kn[2]}"),
        "roofline_verify": roof("verify", v_gbs, v_bytes, v_us,
                                f"verify call{' (fused append)' if fuse else ''}: {kn[1]} + {kn[2]}"),
        "roofline_flush": roof("flush", f_gbs, f_bytes, f_us,
                               f"flush_kernel<128>, {L} layers x {H} heads in one launch",
                               launches=L * H),
        "roofline_prefill": roof("prefill", p_gbs, p_bytes, p_us,
                                 f"prefill_kernel<128> (whole groups and the rest to the ring "
                                 f"in one launch): one layer's {ctx + 64}-token prompt, {H} heads"),
        "spec_accept": {
            f"batch{sb}": {"kernel": f"row_stats_kernel + part_sums_kernel + accept_kernel: "
                                     f"batch {sb}, gamma {gamma}, vocab {V_SPEC}",
                           "avg_launch_us": round(us, 2), "bytes_per_launch": int(nb),
                           "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                           "bound": "latency (dependent round trips)" if sb == 1 else "hbm"}
            for sb, (us, gbs, nb) in sa.items()},
        "graph_step": graph_line,
        "ctx32k": ctx32k,
        "gqa": gqa,
        "meta16": meta16,
        "topk": topk,
        "samples_dropped": dropped,
        "read_ceiling": read_ceiling,
        "mixed_ceiling": mixed_ceiling,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(line), flush=True)


def measure_graph_steps(torch, cache, x, accept, args, L, H, D, gamma, m, out_d, out_v, dev,
                        stream):
    nq0, nt0, _ = cache.state(0)
    nq, nt = int(nq0[0]), int(nt0[0])
    acc_all = torch.tensor(accept, dtype=torch.int32, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)

    def ops(st):
        for j in range(gamma):
            for layer in range(L):
                cache.append_dev(layer, x["dk"][j, layer], x["dv"][j, layer], stream=st)
                cache.attend_draft_dev(layer, x["qd"][j, layer], out_d, stream=st)
        for layer in range(L):
            cache.rollback_dev(layer, gamma, stream=st)
            cache.append_dev(layer, x["tk"][layer], x["tv"][layer], stream=st)
            cache.attend_verify_dev(layer, x["qv"][layer], out_v, stream=st)
            cache.rollback_dev(layer, gamma, sub=acc, stream=st)
        cache.flush_dev(-1, G, stream=st)

    def mirror(nq, nt, a):
        nbytes = 0
        for _ in range(gamma):
            nt += 1
            nbytes += L * (append_bytes(1, H, D) + draft_bytes(nq, nt, H, D))
        nt += m - gamma
        nbytes += L * (append_bytes(m, H, D) + verify_bytes(nq, nt, H, D, m))
        nt -= gamma - a
        if nt >= G:
            nq, nt = nq + G, nt - G
            nbytes += L * flush_bytes(H, D)
        return nq, nt, nbytes

    cache.to_device_state()
    acc.copy_(acc_all[0:1])
    ops(stream)                                   # one eager step in device mode
    nq, nt, _ = mirror(nq, nt, accept[0])
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        ops(cap)
    n = min(args.steps, len(accept) - 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0
    e0.record(stream)
    for s in range(1, n + 1):
        acc.copy_(acc_all[s:s + 1])
        graph.replay()
        nq, nt, b = mirror(nq, nt, accept[s])
        total += b
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    err = cache.from_device_state()
    dq, dt, _ = cache.state(L - 1)
    assert err == 0 and (int(dq[0]), int(dt[0])) == (nq, nt), (err, dq, dt, nq, nt)
    return {"ms_per_step": round(ms, 4), "steps": n,
            "gbs": round(total / n / (ms * 1e-3) / 1e9, 1),
            "calls_per_step": L * (2 * gamma + 4) + 1,
            "note": "the timed step's calls captured once in a HIP graph (device-mode bookkeeping) "
                    "and replayed; each replay preceded by a 4-byte device copy of the step's "
                    "accepted count"}


def measure_gqa(torch, stream, spin_cycles, dev, ctx=131072, Hkv=8, g=4, mt=4, reps=20):
    """Grouped queries on a Llama-3.1-8B-shaped layer: 8 cached heads shared by 4 query heads
    each (32 query heads), head_dim 128, ctx tokens quantized plus a 64 + mt token tail; the
    draft (32 queries, upper planes) and the mt-token verify (16 query columns per cached head)
    timed over `reps` consecutive calls behind the spin kernel.  Bytes: the cached heads' planes
    and metadata once, the tail, and q / out of every query head."""
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache
    D = 128
    cache = Cache(1, 1, Hkv, D, ctx + 16 * G, 15)
    k, v = synth.kv_device(torch, 1, ctx + 64 + mt, Hkv, D, 4242, 4243, dev,
                           outliers=synth.outlier_channels(Hkv, D, 4244))
    cache.prefill(0, k[:, :ctx + 64].contiguous(), v[:, :ctx + 64].contiguous())
    cache.append(0, k[:, ctx + 64:].contiguous(), v[:, ctx + 64:].contiguous())
    del k, v
    gen = torch.Generator(device=dev).manual_seed(4245)
    qd = (torch.randn((1, Hkv * g, D), generator=gen, device=dev) / math.sqrt(D)).half()
    qv = (torch.randn((1, mt, Hkv * g, D), generator=gen, device=dev) / math.sqrt(D)).half()
    od = torch.empty((1, Hkv * g, D), dtype=torch.float32, device=dev)
    ov = torch.empty((1, mt, Hkv * g, D), dtype=torch.float32, device=dev)
    nt = 64 + mt
    out = {"workload": f"Llama-3.1-8B-shaped layer: {Hkv} cached heads x {g} query heads each, "
                       f"head_dim {D}, ctx {ctx} + {nt}-token tail; verify of {mt} tokens "
                       f"({mt * g} query columns per cached head)"}
    for name, fn, nbytes in (
            ("draft", lambda: cache.attend_draft_gqa(0, qd, g, out=od),
             Hkv * (ctx * (D + 8 * D // G + 8) + nt * 4 * D) + Hkv * g * (2 * D + 4 * D)),
            ("verify", lambda: cache.attend_verify_gqa(0, qv, g, out=ov),
             Hkv * (ctx * (2 * D + 8 * D // G + 8) + nt * 4 * D) + mt * Hkv * g * (2 * D + 4 * D))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        torch.cuda._sleep(spin_cycles)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[f"{name}_us"] = round(us, 2)
        out[f"{name}_bytes"] = int(nbytes)
        out[f"{name}_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        out[f"{name}_frac"] = round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    cache.close()
    return out


def measure_meta16(torch, stream, spin_cycles, dev, name, ctx=131072, H=32, m=7, reps=20,
                   rounds=3):
    """fp16 (scale, offset) metadata against fp32 (scale, zero-point) on one layer of the
    workload: H heads, head_dim 128, ctx tokens quantized plus a 64 + m token tail, in two caches that differ
    only in the metadata format.  The draft and the m-query verify are timed over `reps`
    consecutive calls behind the spin kernel, the two formats alternating for `rounds` rounds;
    the best round of each is reported."""
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache
    D, nt = 128, 64 + m
    k, v = synth.kv_device(torch, 1, ctx + nt, H, D, 5151, 5152, dev,
                           outliers=synth.outlier_channels(H, D, 5153))
    gen = torch.Generator(device=dev).manual_seed(5154)
    qd = (torch.randn((1, H, D), generator=gen, device=dev) / math.sqrt(D)).half()
    qv = (torch.randn((1, m, H, D), generator=gen, device=dev) / math.sqrt(D)).half()
    od = torch.empty((1, H, D), dtype=torch.float32, device=dev)
    ov = torch.empty((1, m, H, D), dtype=torch.float32, device=dev)
    caches = {}
    for fmt, m16 in (("fp32", False), ("fp16", True)):
        c = Cache(1, 1, H, D, ctx + 2 * G, m - 1, meta_fp16=m16)
        c.prefill(0, k[:, :ctx + 64].contiguous(), v[:, :ctx + 64].contiguous())
        c.append(0, k[:, ctx + 64:].contiguous(), v[:, ctx + 64:].contiguous())
        caches[fmt] = c
    del k, v
    out = {"workload": f"one layer of the {name} workload: {H} heads, head_dim {D}, ctx {ctx} + "
                       f"{nt}-token tail, verify of {m} queries; fp32 vs fp16 metadata, best of "
                       f"{rounds} alternating rounds of {reps} calls"}
    best = {}
    for _ in range(rounds):
        for fmt, c in caches.items():
            for name, fn in (("draft", lambda: c.attend_draft(0, qd, out=od)),
                             ("verify", lambda: c.attend_verify(0, qv, out=ov))):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                torch.cuda._sleep(spin_cycles)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
                best[(name, fmt)] = min(us, best.get((name, fmt), us))
    for (name, fmt), us in sorted(best.items()):
        mb = 4 if fmt == "fp16" else 8
        nbytes = draft_bytes(ctx, nt, H, D, mb) if name == "draft" else verify_bytes(ctx, nt, H, D, m, mb)
        out[f"{name}_{fmt}_us"] = round(us, 2)
        out[f"{name}_{fmt}_bytes"] = int(nbytes)
        out[f"{name}_{fmt}_frac"] = round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    for c in caches.values():
        c.close()
    return out


def measure_topk(torch, stream, spin_cycles, dev, name, ctx=131072, H=32, m=7, reps=20,
                 rounds=3):
    """The top-k-bit draft: a 2-layer cache in the split-upper layout (the upper nibble as a
    2-bit top plane and a 2-bit middle plane) against a 2-layer cache in the default layout, on
    the same input (H heads, head_dim 128, ctx tokens quantized plus a 64 + m token tail).
    Timed over `reps` consecutive calls behind the spin kernel, alternating between the two
    layers (each call's bytes are not served from the previous call's cache lines): the 2-bit
    draft (top planes only), the 4-bit draft and the m-query verify on each layout; `rounds`
    alternating rounds, the best of each reported."""
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache
    D, nt = 128, 64 + m
    gen = torch.Generator(device=dev).manual_seed(6154)
    qd = (torch.randn((1, H, D), generator=gen, device=dev) / math.sqrt(D)).half()
    qv = (torch.randn((1, m, H, D), generator=gen, device=dev) / math.sqrt(D)).half()
    od = torch.empty((1, H, D), dtype=torch.float32, device=dev)
    ov = torch.empty((1, m, H, D), dtype=torch.float32, device=dev)
    caches = {lay: Cache(2, 1, H, D, ctx + 2 * G, m - 1, split_upper=(lay == "split"))
              for lay in ("nibble", "split")}
    for layer in range(2):
        k, v = synth.kv_device(torch, 1, ctx + nt, H, D, 6151 + 10 * layer, 6152 + 10 * layer,
                               dev, outliers=synth.outlier_channels(H, D, 6153 + layer))
        for c in caches.values():
            c.prefill(layer, k[:, :ctx + 64].contiguous(), v[:, :ctx + 64].contiguous())
            c.append(layer, k[:, ctx + 64:].contiguous(), v[:, ctx + 64:].contiguous())
        del k, v
    calls = [("draft2", "split", lambda c, l: c.attend_draft_bits(l, qd, 2, out=od)),
             ("draft4", "split", lambda c, l: c.attend_draft(l, qd, out=od)),
             ("verify", "split", lambda c, l: c.attend_verify(l, qv, out=ov)),
             ("draft4", "nibble", lambda c, l: c.attend_draft(l, qd, out=od)),
             ("verify", "nibble", lambda c, l: c.attend_verify(l, qv, out=ov))]
    best = {}
    for _ in range(rounds):
        for call, lay, fn in calls:
            c = caches[lay]
            for i in range(4):
                fn(c, i & 1)
            torch.cuda.synchronize()
            torch.cuda._sleep(spin_cycles)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                fn(c, i & 1)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            best[(call, lay)] = min(us, best.get((call, lay), us))
    out = {"workload": f"one layer of the {name} workload at a time (two layers alternating): "
                       f"{H} heads, head_dim {D}, ctx {ctx} + {nt}-token tail, verify of {m} "
                       f"queries; split-upper vs default layout, best of {rounds} rounds of "
                       f"{reps} calls"}
    for (call, lay), us in sorted(best.items()):
        if call == "verify":
            nbytes = verify_bytes(ctx, nt, H, D, m)
        else:
            nbytes = draft_bytes(ctx, nt, H, D, bits=2 if call == "draft2" else 4)
        key = f"{call}_{lay}"
        out[f"{key}_us"] = round(us, 2)
        out[f"{key}_bytes"] = int(nbytes)
        out[f"{key}_frac"] = round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    for c in caches.values():
        c.close()
    return out


def measure_read_ceiling(torch, stream, call_bytes=None):
    """The practical HBM read rate of this device: a plain grid-stride streaming-read kernel
    (16-byte non-temporal loads, eight in flight per lane; libqs_readprobe.so) over 2 GiB, the
    best of 4, 8 and 12 waves per compute unit, 20 timed launches each.  With call_bytes
    ({name: bytes}), the same kernel (at the best wave count) also reads each call's byte count
    once per launch: the streaming rate a call of that size could reach, ramp and drain
    included."""
    import ctypes
    path = os.path.join(ROOT, "hierarchical_quantized_kv_amd", "libqs_readprobe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: run python -m hierarchical_quantized_kv_amd.build_lib")
    lib = ctypes.CDLL(path)
    lib.qs_probe_stream_read.restype = ctypes.c_int
    lib.qs_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_float)]
    buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = buf.numel() // 16 * 16
    best = None
    for bpc in (1, 2, 3):
        us = ctypes.c_float()
        rc = lib.qs_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                      ctypes.c_void_p(sink.data_ptr()), bpc, 20,
                                      ctypes.c_void_p(stream.cuda_stream), ctypes.byref(us))
        if rc != 0:
            raise RuntimeError(f"qs_probe_stream_read failed with HIP error {rc}")
        gbs = nbytes / (us.value * 1e-6) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, bpc, us.value)
    at_size = {}
    for name, nb in (call_bytes or {}).items():
        nb = min(int(nb), buf.numel()) // 16 * 16
        us = ctypes.c_float()
        rc = lib.qs_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nb,
                                      ctypes.c_void_p(sink.data_ptr()), best[1], 20,
                                      ctypes.c_void_p(stream.cuda_stream), ctypes.byref(us))
        if rc != 0:
            raise RuntimeError(f"qs_probe_stream_read failed with HIP error {rc}")
        gbs = nb / (us.value * 1e-6) / 1e9
        at_size[name] = {"bytes": nb, "avg_launch_us": round(us.value, 2), "gbs": round(gbs, 1),
                         "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del buf
    out = {"gbs": round(best[0], 1), "frac_of_peak": round(best[0] / PEAK_HBM_GBS, 4),
           "kernel": f"grid-stride streaming read, 16 B non-temporal loads, 8 in flight per lane, "
                     f"{4 * best[1]} waves per CU",
           "bytes_per_launch": nbytes, "avg_launch_us": round(best[2], 2)}
    if at_size:
        out["at_call_size"] = at_size
    return out


def measure_mixed_ceiling(torch, stream, out_mib=1024):
    """The practical rate of read + write streams on this device: plain grid-stride kernels
    (16-byte non-temporal loads and stores, libqs_readprobe.so) writing out_mib MiB while reading
    1 or 2 times as much (a copy; about the 1.9 : 1 read / write ratio of the flush and prefill
    kernels), best of 4, 8 and 12 waves per compute unit, 20 timed launches each.  Rates count
    read + written bytes."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_quantized_kv_amd", "libqs_readprobe.so"))
    lib.qs_probe_stream_mix.restype = ctypes.c_int
    lib.qs_probe_stream_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    out_bytes = out_mib << 20
    src = torch.zeros(2 * out_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(out_bytes, dtype=torch.uint8, device="cuda")
    res = {}
    for rpw, name in ((1, "copy"), (2, "read2_write1")):
        best = None
        for bpc in (1, 2, 3):
            us = ctypes.c_float()
            rc = lib.qs_probe_stream_mix(ctypes.c_void_p(src.data_ptr()),
                                         ctypes.c_void_p(dst.data_ptr()), out_bytes, rpw, bpc,
                                         20, ctypes.c_void_p(stream.cuda_stream), ctypes.byref(us))
            if rc != 0:
                raise RuntimeError(f"qs_probe_stream_mix failed with HIP error {rc}")
            gbs = (rpw + 1) * out_bytes / (us.value * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, bpc, us.value)
        res[f"{name}_gbs"] = round(best[0], 1)
        res[f"{name}_frac_of_peak"] = round(best[0] / PEAK_HBM_GBS, 4)
        res[f"{name}_waves_per_cu"] = 4 * best[1]
    del src, dst
    res["kernel"] = (f"grid-stride streams: 16 B non-temporal loads and stores, {out_mib} MiB "
                     f"written, 1x or 2x as much read")
    return res


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_profile_path(config):
    return os.path.join(PROFILES, f"hbm_traffic_{'lwm128k' if config == 4 else 'llama32k'}.md")


def load_traffic(config):
    """HBM bytes per launch measured by the counter profile of this workload, or None when the
    kernels have changed since the counters were taken."""
    path = traffic_profile_path(config)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    out = {}
    for kind in ("draft", "verify", "flush", "prefill"):
        mm = re.search(rf"traffic_{kind}_bytes: (\d+)", text)
        if mm:
            out[kind] = int(mm.group(1))
    return out


def _counter_rows(folder):
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {folder}, found {files}")
    return list(csv.DictReader(open(files[0])))


def write_traffic_summary(fetch_dir, write_dir, args):
    """Per-launch HBM traffic of the hot kernels from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by the ratio of the known byte count of the calibration copy to what the counter
    read for it.  The flush launch is normalised per (layer, head) half it quantizes."""
    copy_kib = args.calibration_copy_mib * 1024
    if copy_kib <= 0:
        raise SystemExit("--traffic-summary needs --calibration-copy-mib (the size the runs used)")
    res = {}
    for cname, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(folder) if r["Counter_Name"] == cname]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"{cname}: no calibration copy dispatch in {folder}")
        factor = copy_kib / max(copies)
        per = {}
        for kind, kname in KERNELS.items():
            sel = [r for r in rows if kname in r["Kernel_Name"].replace("qs::", "")]
            if not sel:
                continue
            vals = [float(r["Counter_Value"]) * factor * 1024 for r in sel]
            if kind == "flush":   # one unit = one (layer, head) half: two 256-thread workgroups
                units = [int(r["Grid_Size"]) // (2 * 256) for r in sel]
                per[kind] = (sum(vals) / sum(units), len(sel))
            else:
                per[kind] = (sum(vals) / len(vals), len(sel))
        res[cname] = (factor, max(copies), per)
    fetch, write = res["FETCH_SIZE"], res["WRITE_SIZE"]
    lines = [
        f"# HBM traffic per launch: {CONFIGS[args.config]['name']} "
        f"(32 heads x head_dim 128, ctx {CONFIGS[args.config]['ctx']})",
        "",
        "Made by (on the GPU, from the repository root; `cd /tmp && export TMPDIR=/tmp` style "
        "temp setup aside):",
        "",
        "```",
        f"timeout -s KILL 200 rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "
        f"\"attn_kernel|combine_kernel|flush_kernel|prefill_kernel|copy\" -d {fetch_dir} -o run "
        f"--output-format csv -- python -u bench.py --config {args.config} --layers 2 --steps 1 "
        f"--warmup 0 --flush-reps 2 --no-cpu-baseline --no-graph --no-gqa --no-meta16 --no-ctx32k "
        f"--no-topk --calibration-copy-mib {args.calibration_copy_mib}",
        f"timeout -s KILL 200 rocprofv3 --pmc WRITE_SIZE (same arguments, -d {write_dir})",
        f"python bench.py --config {args.config} --calibration-copy-mib "
        f"{args.calibration_copy_mib} --traffic-summary {fetch_dir} {write_dir}",
        "```",
        "",
        f"Calibration: one device-to-device copy of {args.calibration_copy_mib} MiB "
        f"(`__amd_rocclr_copyBuffer`) reads and writes {copy_kib} KiB.  The counters read "
        f"FETCH_SIZE {fetch[1]:.0f} KiB (factor {fetch[0]:.4f}) and WRITE_SIZE {write[1]:.0f} KiB "
        f"(factor {write[0]:.4f}) for it; every kernel's counts below are scaled by these factors.",
        "",
        "| kernel | dispatches | read bytes | written bytes | total bytes |",
        "|---|---|---|---|---|",
    ]
    out = {}
    for kind in ("draft", "verify", "combine", "flush", "prefill"):
        if kind not in fetch[2] or kind not in write[2]:
            continue
        rd, n = fetch[2][kind]
        wr, _ = write[2][kind]
        unit = " per (layer, head) half" if kind == "flush" else ""
        lines.append(f"| {KERNELS[kind]}{unit} | {n} | {rd:.0f} | {wr:.0f} | {rd + wr:.0f} |")
        out[kind] = rd + wr
    lines += ["", "Machine-read by bench.py (the figures go null once the kernel source changes):",
              "", "```", f"kernel_source_sha256: {kernel_source_hash()}"]
    for kind, v in out.items():
        lines.append(f"traffic_{kind}_bytes: {int(round(v))}")
    lines += ["```", ""]
    os.makedirs(PROFILES, exist_ok=True)
    path = traffic_profile_path(args.config)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(path)


def _oracle_round(k, v, ctx, D, gamma, heads, barrier=None):
    """One speculation round of the CPU oracle over `heads` of the sample (gamma draft calls,
    each after appending one token, then rollback, gamma+1 appended tokens and one verify
    call); the prefill is not timed.  Returns (draft seconds, verify seconds)."""
    from oracle import OracleCache
    from hierarchical_quantized_kv_amd import synth

    H = len(heads)
    k_all = k
    k, v = np.ascontiguousarray(k[:, :, heads]), np.ascontiguousarray(v[:, :, heads])
    c = OracleCache(1, 1, H, D, G, ctx + 16 * G, gamma)
    for pos in range(0, ctx, G):
        c.append(0, k[:, pos:pos + G], v[:, pos:pos + G])
        c.flush(0)
    nt = 64 - gamma - 1
    m = gamma + 1
    c.append(0, k[:, ctx:ctx + nt], v[:, ctx:ctx + nt])
    HS = k_all.shape[2]  # queries are drawn for all sampled heads, then split by thread
    qd = [np.ascontiguousarray(synth.queries_host(1, None, HS, D, 10 + j)[:, heads])
          for j in range(gamma)]
    qv = np.ascontiguousarray(synth.queries_host(1, m, HS, D, 2)[:, :, heads])
    if barrier is not None:
        barrier.wait()
    t0 = time.perf_counter()
    for j in range(gamma):
        c.append(0, k[:, ctx + nt + j:ctx + nt + j + 1], v[:, ctx + nt + j:ctx + nt + j + 1])
        c.attend_draft(0, qd[j])
    t_d = time.perf_counter() - t0
    c.rollback(0, [gamma])
    c.append(0, k[:, ctx + nt:ctx + nt + m], v[:, ctx + nt:ctx + nt + m])
    t1 = time.perf_counter()
    c.attend_verify(0, qv)
    return t_d, time.perf_counter() - t1


def cpu_baseline(inputs, ctx, D, gamma, threads=1):
    """The CPU oracle, as it is, on a bounded sample of the same workload: layer 0 restricted to
    its first CPU_SAMPLE_HEADS heads, one speculation round.  With threads > 1 the heads are
    dealt to that many host threads (the oracle's C calls release the GIL), each running the
    same round on its own oracle instance, started together; the wall time is the slowest."""
    import threading

    import oracle

    oracle.build(force=False)
    k, v = inputs
    H = k.shape[2]  # the sampled heads
    threads = max(1, min(threads, H))
    nt = 64 - gamma - 1
    m = gamma + 1
    nb = sum(draft_bytes(ctx, nt + 1 + j, H, D) for j in range(gamma))
    nb_v = verify_bytes(ctx, nt + m, H, D, m)
    groups = [list(range(t, H, threads)) for t in range(threads)]
    res = [None] * threads
    barrier = threading.Barrier(threads) if threads > 1 else None

    def run(t):
        res[t] = _oracle_round(k, v, ctx, D, gamma, groups[t], barrier)

    if threads == 1:
        run(0)
    else:
        ts = [threading.Thread(target=run, args=(t,)) for t in range(threads)]
        for th in ts:
            th.start()
        for th in ts:
            th.join()
    t_d = max(r[0] for r in res)
    t_v = max(r[1] for r in res)
    how = "single-threaded" if threads == 1 else f"{threads} host threads, heads dealt round-robin"
    aff, ncpu = host_cpus()
    return {"value": round((nb + nb_v) / (t_d + t_v) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cpus_available": aff, "host_cpus_reported": ncpu, "kind": "oracle",
            "sample": f"layer 0, heads 0..{H - 1} of the same workload at ctx {ctx}: one "
                      f"speculation round = {gamma} draft calls ({t_d:.2f}s) + one {m}-query "
                      f"verify call ({t_v:.2f}s), fp64 oracle, {how}; GB/s = algorithmic bytes "
                      f"of those calls / their time"}


if __name__ == "__main__":
    main()
