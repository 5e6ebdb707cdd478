"""Randomized GPU parity: seeded random configurations (head_dim, batch across the three argument
buckets, heads, gamma_max, draft offset, metadata format, key distribution) driven through random
but valid sequences of the cache's verbs -- prefill of ragged prompts, appends, drafts, fused
append + draft, verifies of 1 .. min(gamma_max + 1, nt) queries, grouped-query draft and verify,
device-mode draft and verify (counters taken to the arena and back), rollbacks, flushes -- with
every attention output compared with the CPU oracle (max abs 2e-3) and the planes, metadata,
ring slots and counters compared bit for bit at the end.

QS_RANDOM_CASES sets the number of seeds (default 16).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import synth
from lockstep import Lockstep, log

pytestmark = pytest.mark.gpu
G = 128
CASES = int(os.environ.get("QS_RANDOM_CASES", "16"))


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def _kv(rng, B, n, H, D, dist):
    k, v = synth.kv_host(B, n, H, D, int(rng.integers(1 << 30)), int(rng.integers(1 << 30)),
                         dist_k=dist)
    return torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()


def _q(rng, B, m, H, D):
    return torch.from_numpy(synth.queries_host(B, m, H, D, int(rng.integers(1 << 30)),
                                               float(rng.choice([0.5, 1.0, 3.0])))).cuda()


@pytest.mark.parametrize("seed", range(CASES))
def test_random_rounds_match_the_oracle(seed):
    rng = np.random.default_rng(70000 + seed)
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([1, 2, 3, 8, 9, 12]))
    H = int(rng.integers(1, 5))
    gmax = int(rng.integers(0, 16))
    off = int(rng.choice([0, 8]))
    m16 = bool(rng.integers(0, 2))
    dist = str(rng.choice(["normal", "student_t3"]))
    # up to 70 groups: with many (sequence, head) pairs a worker then takes several groups
    T = G * int(rng.choice([2, 3, 4, 6, 16, 40, 70]))
    log(f"case: random seed {seed}: D={D} B={B} H={H} gamma_max={gmax} off={off} "
        f"fp16 metadata {m16} keys {dist} max_ctx {T}")
    ls = Lockstep(1, B, H, D, T, gmax, draft_offset=off, tag=f"rand{seed}", meta_fp16=m16)
    orc = ls.orc[0]

    lens = [int(rng.integers(0, T - G + 1)) for _ in range(B)]
    if max(lens) > 0:
        k, v = _kv(rng, B, max(lens), H, D, dist)
        ls.prefill(0, k, v, lens)
    ops = []
    for _ in range(14):
        nq, nt, _ = orc.state(0)
        op = str(rng.choice(["append", "append", "draft", "fused", "verify", "gqa", "dev",
                             "rollback", "flush"]))
        if op in ("append", "fused"):
            n = [int(rng.integers(0, min(2 * G - int(t), 9) + 1)) for t in nt]
            if max(n) == 0:
                continue
            if op == "fused" and any(int(a) + int(t) + c == 0 for a, t, c in zip(nq, nt, n)):
                op = "append"
            k, v = _kv(rng, B, max(n), H, D, dist)
            if op == "append":
                ls.append(0, k, v, n)
            else:
                q = _q(rng, B, None, H, D)
                out = ls.gpu.append_attend_draft(0, k, v, q, n=n)
                orc.append(0, ls._host_heads(k, 2), ls._host_heads(v, 2), n)
                ref = orc.attend_draft(0, ls._host_heads(q, 1))
                torch.cuda.synchronize()
                ls._cmp_out(out, ref, "fused draft")
        elif op == "draft":
            if any(int(a) + int(t) == 0 for a, t in zip(nq, nt)):
                continue
            ls.draft(0, _q(rng, B, None, H, D), sm_scale=float(rng.choice([0.7, 1.0])))
        elif op == "verify":
            top = min(gmax + 1, int(min(nt)))
            if top < 1:
                continue
            m = int(rng.integers(1, top + 1))
            ls.verify(0, _q(rng, B, m, H, D))
        elif op == "gqa":   # g query heads per cached head; the oracle once per r
            if any(int(a) + int(t) == 0 for a, t in zip(nq, nt)):
                continue
            g = int(rng.integers(1, min(4, gmax + 1) + 1))   # g query columns <= gamma_max + 1
            mt = int(rng.integers(0, min((gmax + 1) // g, int(min(nt))) + 1))
            qg = _q(rng, B, None, H * g, D)
            out_d = ls.gpu.attend_draft_gqa(0, qg, g)
            out_v = None
            if mt >= 1:
                qgv = _q(rng, B, mt, H * g, D)
                out_v = ls.gpu.attend_verify_gqa(0, qgv, g)
            torch.cuda.synchronize()
            for r in range(g):
                heads = [h * g + r for h in range(H)]
                ls._cmp_out(out_d[:, heads], orc.attend_draft(0, qg[:, heads].cpu().numpy()),
                            f"gqa draft g={g} r={r}")
                if out_v is not None:
                    ls._cmp_out(out_v[:, :, heads],
                                orc.attend_verify(0, qgv[:, :, heads].contiguous().cpu().numpy()),
                                f"gqa verify g={g} m={mt} r={r}")
        elif op == "dev":   # device-mode draft and verify, the counters back on the host after
            if any(int(a) + int(t) == 0 for a, t in zip(nq, nt)):
                continue
            m = int(rng.integers(0, min(gmax + 1, int(min(nt))) + 1))
            qd = _q(rng, B, None, H, D)
            od = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
            ls.gpu.to_device_state()
            ls.gpu.attend_draft_dev(0, qd, od)
            if m >= 1:
                qv = _q(rng, B, m, H, D)
                ov = torch.empty((B, m, H, D), dtype=torch.float32, device="cuda")
                ls.gpu.attend_verify_dev(0, qv, ov)
            assert ls.gpu.from_device_state() == 0
            torch.cuda.synchronize()
            ls._cmp_out(od, orc.attend_draft(0, ls._host_heads(qd, 1)), "device draft")
            if m >= 1:
                ls._cmp_out(ov, orc.attend_verify(0, ls._host_heads(qv, 2)), "device verify")
            ls.check_state(0)
        elif op == "rollback":
            ls.rollback(0, [int(rng.integers(0, int(t) + 1)) for t in nt])
        else:  # flush, unless a sequence that would be selected has no room left
            if any(int(t) >= G and int(a) + G > T for a, t in zip(nq, nt)):
                continue
            ls.flush(0)
        ops.append(op)
    ls.check_planes(0)
    log(f"rand{seed}: ops {' '.join(ops)}; max abs {ls.max_abs:.3e} max rel {ls.max_rel:.3e}")
