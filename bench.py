"""Benchmark of the decode-attention hot path of the hierarchical INT8 KV cache on one GPU.

Workload (default): LWM-128k-shaped cache, 32 layers x 32 heads x head_dim 128, batch 1, 131072
prefilled tokens (1024 quantized groups per head) plus a 64-token fp16 tail, keys with 1 % of
channels scaled x8.  One step is one speculation round over all layers:
  gamma = 6 draft steps (per layer: append 1 token, draft attention),
  per layer: rollback gamma, append gamma+1 target tokens, verify attention (7 queries),
  acceptance a ~ Bernoulli(0.9) until first reject, rollback gamma - a, then one flush call.
Inputs are seeded synthetic fp16 tensors resident in HBM before timing starts.

Prints one JSON line: value = algorithmic HBM bytes of the step / step time (GB/s).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step and HBM GB/s (draft & verify) at 32k/128k ctx"
PEAK_HBM_GBS = 8000.0
G = 128

CONFIGS = {
    3: dict(name="Llama-2-7B-32K-shaped full stack", layers=32, heads=32, D=128, ctx=32768,
            gamma=4),
    4: dict(name="LWM-128k-shaped", layers=32, heads=32, D=128, ctx=131072, gamma=6),
}


def draft_bytes(nq, nt, H, D):
    """Algorithmic bytes of one draft call: upper key/value planes + fp32 (s, z) metadata of
    every quantized token-head, the fp16 tail, the query and the fp32 output."""
    per_tok = D // 2 + D // 2 + 8 * D // G + 8
    return H * (nq * per_tok + nt * 4 * D + 2 * D + 4 * D)


def verify_bytes(nq, nt, H, D, m):
    per_tok = D + D + 8 * D // G + 8
    return H * (nq * per_tok + nt * 4 * D + m * (2 * D + 4 * D))


def flush_bytes(H, D):
    """One flushed G-token half per head: fp16 keys and values read, both planes of both
    written, key (s, z) per channel and value (s, z) per token written."""
    return H * (G * D * 2 * 2 + 2 * G * D + 8 * D + 8 * G)


def append_bytes(n, H, D):
    return 2 * n * H * D * 2 * 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=4, choices=sorted(CONFIGS))
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4)
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this size first (reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from hierarchical_quantized_kv_amd import synth
    from hierarchical_quantized_kv_amd.binding import Cache

    cfg = CONFIGS[args.config]
    L = args.layers or cfg["layers"]
    H, D, ctx, gamma = cfg["heads"], cfg["D"], cfg["ctx"], cfg["gamma"]
    m = gamma + 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    max_ctx = ctx + 16 * G
    print(f"bench: config {args.config} ({cfg['name']}), {L} layers, ctx {ctx}", file=sys.stderr,
          flush=True)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 19  # fp16 elements
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cache = Cache(L, 1, H, D, max_ctx, gamma)
    t0 = time.time()
    cpu_inputs = None
    for layer in range(L):
        out_ch = synth.outlier_channels(H, D, synth.seed_for(args.config, layer, "outlier"))
        k, v = synth.kv_device(torch, 1, ctx + 64, H, D,
                               synth.seed_for(args.config, layer, "k"),
                               synth.seed_for(args.config, layer, "v"), dev, outliers=out_ch)
        for pos in range(0, ctx, G):
            cache.append(layer, k[:, pos:pos + G], v[:, pos:pos + G])
            cache.flush(layer)
        cache.append(layer, k[:, ctx:].contiguous(), v[:, ctx:].contiguous())
        if layer == 0 and not args.no_cpu_baseline:
            hs = list(range(args.cpu_heads))
            cpu_inputs = (k[:, :, hs].cpu().numpy(), v[:, :, hs].cpu().numpy())
        del k, v
    torch.cuda.synchronize()
    print(f"bench: prefill done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # per-step inputs, generated up front (resident in HBM before timing)
    n_steps = args.warmup + args.steps
    gen = torch.Generator(device=dev).manual_seed(12345)
    rng = np.random.Generator(np.random.PCG64(synth.seed_for(args.config, 0, "accept")))
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
    stream = torch.cuda.current_stream()

    ev = {"draft": [], "verify": []}
    step_bytes = []

    def run_step(s, timed):
        x = steps_in[s]
        nbytes = 0
        for j in range(gamma):
            for layer in range(L):
                cache.append(layer, x["dk"][j, layer], x["dv"][j, layer])
                nq, nt, _ = cache.state(layer)
                nbytes += append_bytes(1, H, D) + draft_bytes(int(nq[0]), int(nt[0]), H, D)
                if timed:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                cache.attend_draft(layer, x["qd"][j, layer], out=out_d)
                if timed:
                    e1.record(stream)
                    ev["draft"].append((e0, e1, draft_bytes(int(nq[0]), int(nt[0]), H, D)))
        for layer in range(L):
            cache.rollback(layer, [gamma])
            cache.append(layer, x["tk"][layer], x["tv"][layer])
            nq, nt, _ = cache.state(layer)
            vb = verify_bytes(int(nq[0]), int(nt[0]), H, D, m)
            nbytes += append_bytes(m, H, D) + vb
            if timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            cache.attend_verify(layer, x["qv"][layer], out=out_v)
            if timed:
                e1.record(stream)
                ev["verify"].append((e0, e1, vb))
            cache.rollback(layer, [gamma - accept[s]])
        flushed = cache.flush(-1)
        nbytes += int(flushed[0]) * L * flush_bytes(H, D)
        return nbytes

    for s in range(args.warmup):
        run_step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, n_steps):
        step_bytes.append(run_step(s, True))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    total_bytes = sum(step_bytes)
    value = total_bytes / elapsed / 1e9

    def summarize(kind):
        t = [a.elapsed_time(b) * 1e3 for a, b, _ in ev[kind]]   # us
        by = [n for _, _, n in ev[kind]]
        mean_us = float(np.mean(t))
        return mean_us, float(np.mean(by)) / (mean_us * 1e-6) / 1e9, float(np.mean(by))

    d_us, d_gbs, d_bytes = summarize("draft")
    v_us, v_gbs, v_bytes = summarize("verify")

    cpu = None
    if cpu_inputs is not None:
        cpu = cpu_baseline(cpu_inputs, ctx, D, gamma, args.cpu_heads)

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
                   "batch": 1, "group": G},
        "draft_us_per_layer": round(d_us, 2),
        "draft_gbs": round(d_gbs, 1),
        "verify_us_per_layer": round(v_us, 2),
        "verify_gbs": round(v_gbs, 1),
        "roofline": {"bound": "hbm", "kernel": "draft attention (attn_kernel<128, draft> + combine)",
                     "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(d_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(d_bytes), "avg_launch_us": round(d_us, 2)},
        "roofline_verify": {"bound": "hbm", "achieved": round(v_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(v_gbs / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": int(v_bytes), "avg_launch_us": round(v_us, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inputs, ctx, D, gamma, n_heads):
    """The CPU oracle, as it is, on a bounded sample of the same workload: layer 0 restricted to
    the first n_heads heads; one draft call and one verify call timed (single thread)."""
    import oracle
    from oracle import OracleCache
    from hierarchical_quantized_kv_amd import synth

    oracle.build(force=False)
    k, v = inputs
    H = n_heads
    c = OracleCache(1, 1, H, D, G, ctx + 16 * G, gamma)
    for pos in range(0, ctx, G):
        c.append(0, k[:, pos:pos + G], v[:, pos:pos + G])
        c.flush(0)
    c.append(0, k[:, ctx:ctx + 64], v[:, ctx:ctx + 64])
    q = synth.queries_host(1, None, H, D, 1)
    t0 = time.perf_counter()
    c.attend_draft(0, q)
    t_d = time.perf_counter() - t0
    m = gamma + 1
    c.append(0, k[:, ctx + 64 - m:ctx + 64], v[:, ctx + 64 - m:ctx + 64])
    qv = synth.queries_host(1, m, H, D, 2)
    t0 = time.perf_counter()
    c.attend_verify(0, qv)
    t_v = time.perf_counter() - t0
    nb = draft_bytes(ctx, 64, H, D) + verify_bytes(ctx, 64 + m, H, D, m)
    return {"value": round(nb / (t_d + t_v) / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"layer 0, heads 0..{H - 1} of the same workload: one draft call "
                      f"({t_d:.2f}s) and one {m}-query verify call ({t_v:.2f}s) at ctx {ctx}, "
                      f"single-threaded fp64 oracle; GB/s = algorithmic bytes of those calls / time"}


if __name__ == "__main__":
    main()
