"""Device mode on the GPU: a whole speculation round -- gamma draft steps over every layer, the
verify pass, the accept / correct step, the rollback by the accepted count and the flush -- is
captured once in a HIP graph (through torch.cuda.CUDAGraph) and replayed round after round, with
fresh inputs written between the replays and the counters advancing on the device.  Every
replay is checked against the fp64 oracle driven through the same round on the CPU; at the end
the counters, planes, metadata and tail are compared bit for bit.

The round follows the cache-manager and verification-loop listings of the QuantSpec Guide (a
speculative buffer rolled back after verification) and the Pith review's "What carries the
argument": before verify the gamma draft tokens are rolled back and the gamma + 1 target tokens
appended; after the accept step the gamma - a rejected ones are rolled back; the flush
quantizes one G half once the tail holds G tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import binding, synth
from hierarchical_quantized_kv_amd.binding import Cache, spec_accept, spec_workspace_bytes
from lockstep import ATOL, Lockstep, log

pytestmark = pytest.mark.gpu
G = 128


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


class Round:
    """Static device buffers of one speculation round and the calls that make it up."""

    def __init__(self, cache, gamma, vocab):
        L, B, H, D = cache.L, cache.B, cache.H, cache.D
        dev = torch.device("cuda")
        f16, f32, i32 = torch.float16, torch.float32, torch.int32
        self.c, self.gamma, self.V = cache, gamma, vocab
        self.dk = torch.zeros((gamma, B, 1, H, D), dtype=f16, device=dev)
        self.dv = torch.zeros_like(self.dk)
        self.dq = torch.zeros((gamma, B, H, D), dtype=f16, device=dev)
        self.vk = torch.zeros((B, gamma + 1, H, D), dtype=f16, device=dev)
        self.vv = torch.zeros_like(self.vk)
        self.vq = torch.zeros_like(self.vk)
        self.out_d = torch.zeros((L, gamma, B, H, D), dtype=f32, device=dev)
        self.out_v = torch.zeros((L, B, gamma + 1, H, D), dtype=f32, device=dev)
        self.t = torch.zeros((B, gamma + 1, vocab), dtype=f32, device=dev)
        self.d = torch.zeros((B, gamma, vocab), dtype=f32, device=dev)
        self.x = torch.zeros((B, gamma), dtype=i32, device=dev)
        self.u = torch.zeros((B, gamma + 1), dtype=f32, device=dev)
        self.n_acc = torch.zeros(B, dtype=i32, device=dev)
        self.nxt = torch.zeros(B, dtype=i32, device=dev)
        self.ws = torch.empty(spec_workspace_bytes(B, gamma, vocab), dtype=torch.uint8, device=dev)

    def ops(self, stream):
        c, g = self.c, self.gamma
        for i in range(g):                      # draft step i over every layer
            for l in range(c.L):
                c.append_dev(l, self.dk[i], self.dv[i], stream=stream)
                c.attend_draft_dev(l, self.dq[i], self.out_d[l, i], stream=stream)
        for l in range(c.L):                    # verify: the target's gamma + 1 tokens
            c.rollback_dev(l, g, stream=stream)
            c.append_dev(l, self.vk, self.vv, stream=stream)
            c.attend_verify_dev(l, self.vq, self.out_v[l], stream=stream)
        spec_accept(self.t, self.d, self.x, self.u, workspace=self.ws, stream=stream,
                    n_out=self.n_acc, next_out=self.nxt)
        c.rollback_dev(-1, g, sub=self.n_acc, stream=stream)   # keep a + 1 of the gamma + 1
        c.flush_dev(-1, G, stream=stream)

    def fill(self, rng):
        """Fresh seeded inputs: K/V ~ N(0,1), q ~ N(0,1)/sqrt(D), logits as in the accept tests."""
        B, H, D, g, V = self.c.B, self.c.H, self.c.D, self.gamma, self.V
        h = {}
        for name, shape, scale in (("dk", self.dk.shape, 1.0), ("dv", self.dv.shape, 1.0),
                                   ("dq", self.dq.shape, D ** -0.5), ("vk", self.vk.shape, 1.0),
                                   ("vv", self.vv.shape, 1.0), ("vq", self.vq.shape, D ** -0.5)):
            h[name] = (rng.standard_normal(shape) * scale).astype(np.float16)
            getattr(self, name).copy_(torch.from_numpy(h[name]))
        t = rng.normal(0, 2.0, (B, g + 1, V)).astype(np.float32)
        d = (t[:, :g] + rng.normal(0, 1.0, (B, g, V))).astype(np.float32)
        e = np.exp(d - d.max(-1, keepdims=True))
        cdf = np.cumsum(e / e.sum(-1, keepdims=True), -1)
        x = np.minimum((cdf < rng.random((B, g, 1))).sum(-1), V - 1).astype(np.int32)
        u = rng.random((B, g + 1)).astype(np.float32)
        for name, a in (("t", t), ("d", d), ("x", x), ("u", u)):
            h[name] = a
            getattr(self, name).copy_(torch.from_numpy(a))
        return h


def oracle_round(ls, h, n_gpu, gamma, rnd):
    """The same round on the oracle; attention compared with the graph's outputs."""
    out_d, out_v = h["out_d"], h["out_v"]
    for i in range(gamma):
        for l in ls.layers:
            ls.orc[l].append(0, h["dk"][i], h["dv"][i])
            ref = ls.orc[l].attend_draft(0, h["dq"][i])
            ls._cmp_out(torch.from_numpy(out_d[l, i]), ref, f"round {rnd} draft {i} L{l}")
    for l in ls.layers:
        ls.orc[l].rollback(0, [gamma] * ls.B)
        ls.orc[l].append(0, h["vk"], h["vv"])
        ref = ls.orc[l].attend_verify(0, h["vq"])
        ls._cmp_out(torch.from_numpy(out_v[l]), ref, f"round {rnd} verify L{l}")
    n_o, nxt_o, mg = oracle.spec_accept(h["t"], h["d"], h["x"], h["u"])
    n_g, nxt_g = n_gpu
    close = mg < 1e-5
    assert np.array_equal(n_g[~close], n_o[~close]) and np.array_equal(nxt_g[~close], nxt_o[~close])
    for l in ls.layers:          # the oracle follows the device's accepted counts
        ls.orc[l].rollback(0, [gamma - int(a) for a in n_g])
        ls.orc[l].flush(0, G)
    return n_g


@pytest.mark.parametrize("B,H,D,lens,m16", [
    (2, 4, 128, (3 * G + 120, 5 * G + 126), False),      # the 8-sequence argument bucket
    (1, 8, 128, (2 * G + 127,), False),                   # the 1-sequence bucket
    # the 64-sequence bucket at D = 64; sequences 0, 4, 8 start with an empty quantized tier
    (9, 2, 64, tuple(G * (i % 4) + 122 + i % 5 for i in range(9)), False),
    (2, 4, 128, (3 * G + 120, 5 * G + 126), True),       # fp16 metadata
])
def test_graph_round_replays_match_oracle(B, H, D, lens, m16):
    L, gamma, V, rounds = 2, 4, 1000, 6
    log(f"case: device-mode graph round B={B} H={H} D={D} prompts={lens} gamma={gamma} "
        f"rounds={rounds} fp16 metadata {m16}")
    ls = Lockstep(L, B, H, D, 16 * G, gamma, tag="graph", meta_fp16=m16)
    n_max = max(lens)
    for l in range(L):
        k, v = synth.kv_device(torch, B, n_max, H, D, 600 + l, 700 + l, "cuda")
        ls.prefill(l, k, v, n=list(lens))
    torch.cuda.synchronize()
    # load every kernel once (a scratch cache of the same shape) before capturing
    warm = Cache(L, B, H, D, 16 * G, gamma, meta_fp16=m16)
    kw, vw = synth.kv_device(torch, B, G + 8, H, D, 1, 2, "cuda")   # every sequence non-empty
    for l in range(L):
        warm.prefill(l, kw, vw)
    warm.to_device_state()
    wr = Round(warm, gamma, V)
    wr.fill(np.random.default_rng(0))
    wr.ops(torch.cuda.current_stream())
    assert warm.from_device_state() == 0
    warm.close()

    rd = Round(ls.gpu, gamma, V)
    ls.gpu.to_device_state()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        rd.ops(cap)
    rng = np.random.default_rng(2025)
    accepted = []
    for r in range(rounds):
        h = rd.fill(rng)
        graph.replay()
        torch.cuda.synchronize()
        h["out_d"] = rd.out_d.cpu().numpy()
        h["out_v"] = rd.out_v.cpu().numpy()
        n_g = (rd.n_acc.cpu().numpy(), rd.nxt.cpu().numpy())
        accepted.append(oracle_round(ls, h, n_g, gamma, r).tolist())
    err = ls.gpu.from_device_state()
    assert err == 0, err
    for l in range(L):
        ls.check_planes(l)
    nq, nt, _ = ls.gpu.state(0)
    log(f"graph: {rounds} replays, accepted per round {accepted}, final nq {nq.tolist()} nt "
        f"{nt.tolist()}, max abs err {ls.max_abs:.2e}")
    # every sequence crossed G tail tokens and flushed at least once
    assert all(int(q) > (n // G) * G for q, n in zip(nq, lens)), (nq, lens)


def test_device_errors_are_flagged_and_leave_the_state():
    """Conditions only the device can see are flagged in the error word, and the sequence keeps
    its counters (and its tail): an append past 2G, a rollback past the tail, a verify with
    m > nt, a flush past max_ctx."""
    L, B, H, D = 1, 2, 2, 64
    log("case: device-mode error word")
    c = Cache(L, B, H, D, 2 * G, 4)
    k, v = synth.kv_device(torch, B, 2 * G, H, D, 5, 6, "cuda")
    c.prefill(0, k, v, n=[2 * G, 0])          # sequence 0 full (nq = max_ctx), sequence 1 empty
    c.append(0, k[:, :10].contiguous(), v[:, :10].contiguous())
    torch.cuda.synchronize()
    tail0 = c.section("tail_k", 0).view(torch.int16).clone()   # bits: unused slots may hold NaNs
    c.to_device_state()
    big = k[:, :2 * G - 5].contiguous(), v[:, :2 * G - 5].contiguous()
    c.append_dev(0, *big)                               # 10 + 251 > 256: flagged, nothing written
    torch.cuda.synchronize()
    assert torch.equal(c.section("tail_k", 0).view(torch.int16), tail0)
    c.rollback_dev(0, 11)                               # 11 > nt = 10
    q = torch.zeros((B, 5, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty((B, 5, H, D), dtype=torch.float32, device="cuda")
    c.attend_verify_dev(0, q, out)                      # m = 5 <= nt = 10: fine
    torch.cuda.synchronize()
    assert c.from_device_state() == binding.DEV_ERR_APPEND | binding.DEV_ERR_ROLLBACK
    nq, nt, hd = c.state(0)
    assert nq.tolist() == [2 * G, 0] and nt.tolist() == [10, 10] and hd.tolist() == [0, 0]
    c.append(0, k[:, :G].contiguous(), v[:, :G].contiguous())   # nt = 138 >= G
    c.to_device_state()
    c.flush_dev(0, G)                                   # sequence 0 is at max_ctx: flagged
    c.attend_verify_dev(0, torch.zeros((B, 5, H, D), dtype=torch.float16, device="cuda"), out)
    sub = torch.tensor([0, G], dtype=torch.int32, device="cuda")
    c.rollback_dev(0, 138 - 3, sub=sub)                 # drops 135 and 7: nt = 3 for both
    c.attend_verify_dev(0, q, out)                      # m = 5 > nt = 3: flagged
    torch.cuda.synchronize()
    assert c.from_device_state() == binding.DEV_ERR_FLUSH | binding.DEV_ERR_ATTEND
    nq, nt, hd = c.state(0)
    assert nq.tolist() == [2 * G, G] and nt.tolist() == [3, 3] and hd.tolist() == [0, G]
    c.close()


def test_pending_operations_and_commit_points():
    """Appends and rollbacks recorded as pending operations give the host verbs' counters and
    ring contents, through every commit point: a fifth pending operation, qs_commit_dev, and
    qs_state_from_device."""
    L, B, H, D = 2, 2, 2, 64
    log("case: device-mode pending operations")
    dev_c, host_c = Cache(L, B, H, D, 4 * G, 4), Cache(L, B, H, D, 4 * G, 4)
    k, v = synth.kv_device(torch, B, G + 8, H, D, 21, 22, "cuda")
    for c in (dev_c, host_c):
        for l in range(L):
            c.prefill(l, k, v, n=[G + 3, 5])
    dev_c.to_device_state()
    for i in range(5):                                  # the fifth commits the first four
        kk, vv = k[:, i:i + 1].contiguous(), v[:, i:i + 1].contiguous()
        dev_c.append_dev(0, kk, vv)
        host_c.append(0, kk, vv)
    dev_c.rollback_dev(0, 2)
    host_c.rollback(0, [2, 2])
    dev_c.commit_dev(0)
    sub = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    dev_c.rollback_dev(1, 1, sub=sub)
    host_c.rollback(1, [0, 1])
    kk, vv = k[:, 5:7].contiguous(), v[:, 5:7].contiguous()
    dev_c.append_dev(1, kk, vv)                         # applies the pending rollback first
    host_c.append(1, kk, vv)
    assert dev_c.from_device_state() == 0               # commits layer 1
    for l in range(L):
        sd, sh = dev_c.state(l), host_c.state(l)
        assert all(np.array_equal(x, y) for x, y in zip(sd, sh)), (l, sd, sh)
        nt, head = sh[1], sh[2]
        for b in range(B):
            slots = [(int(head[b]) + i) % (2 * G) for i in range(int(nt[b]))]
            for name in ("tail_k", "tail_v"):
                got = dev_c.section(name, l)[b][:, slots].view(torch.int16)
                ref = host_c.section(name, l)[b][:, slots].view(torch.int16)
                assert torch.equal(got, ref), (l, b, name)
    assert [dev_c.state(l)[1].tolist() for l in range(L)] == [[6, 8], [5, 6]]
    dev_c.close()
    host_c.close()
