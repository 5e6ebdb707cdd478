"""GPU parity of the speculative accept / correct step (qs_spec_accept) against the fp64 oracle.

Both sides take the accept decisions and the sample from the same uniforms.  The GPU works in
fp32, the oracle in fp64: a decision whose margin (how far u was from flipping it, reported by
the oracle, in units of probability) is below 1e-5 -- the order of the rounding of an fp32
prefix sum over tens of thousands of probabilities -- may come out either way and is only
checked for validity; every other case must match exactly.  Inputs are seeded synthetic logits (the draft's are the target's plus
noise) with drafted tokens drawn from the draft distribution.
"""
import numpy as np
import pytest
import torch

import oracle
from hierarchical_quantized_kv_amd import binding
from lockstep import log

pytestmark = pytest.mark.gpu


def setup_module(_):
    oracle.build(force=False)
    assert torch.cuda.is_available()


def softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def case(seed, B, gamma, V, spread=2.0, noise=1.0):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, spread, (B, gamma + 1, V)).astype(np.float32)
    d = (t[:, :gamma] + rng.normal(0, noise, (B, gamma, V))).astype(np.float32)
    cdf = np.cumsum(softmax(d), axis=-1)
    r = rng.random((B, gamma, 1))
    x = np.minimum((cdf < r).sum(axis=-1), V - 1).astype(np.int32)   # x ~ q by inverse CDF
    u = rng.random((B, gamma + 1)).astype(np.float32)
    return t, d, x, u


def run_gpu(t, d, x, u):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    n, nxt = binding.spec_accept(dev(t), dev(d), dev(x), dev(u))
    return n.cpu().numpy(), nxt.cpu().numpy()


def compare(t, d, x, u, tag):
    n_g, nxt_g = run_gpu(t, d, x, u)
    n_o, nxt_o, mg = oracle.spec_accept(t, d, x, u)
    close = mg < 1e-5
    bad = ~close & ((n_g != n_o) | (nxt_g != nxt_o))
    log(f"{tag}: {len(n_g)} sequences, accepted mean {n_o.mean():.2f}, "
        f"near-boundary {int(close.sum())}, mismatches {int(bad.sum())}")
    assert not bad.any(), (np.nonzero(bad)[0][:5], n_g[bad][:5], n_o[bad][:5], nxt_g[bad][:5],
                           nxt_o[bad][:5])
    # most cases are compared exactly (over a 32000-token vocabulary a sample often lands within
    # 1e-5 of a CDF step, where fp32 prefix sums may choose the neighbour)
    assert close.mean() < 0.4
    V = t.shape[-1]
    assert ((n_g >= 0) & (n_g <= x.shape[1])).all() and ((nxt_g >= 0) & (nxt_g < V)).all()
    return n_o


@pytest.mark.parametrize("B,gamma,V,spread", [(64, 6, 32000, 2.0), (16, 4, 257, 2.0),
                                              (8, 1, 1000, 2.0), (4, 3, 1, 2.0),
                                              (32, 15, 4096, 2.0), (8, 2, 4097, 2.0),
                                              (6, 6, 128256, 4.0)])
def test_matches_oracle(B, gamma, V, spread):
    """Vocabularies of one token, of one 4096-token part plus one token, and of 8 and 32 parts
    (the last ragged); at 128256 tokens the logits are peakier so that most samples land away
    from a CDF step."""
    log(f"case: spec accept B={B} gamma={gamma} V={V} spread={spread}")
    t, d, x, u = case(1000 + V + gamma, B, gamma, V, spread=spread)
    n_o = compare(t, d, x, u, f"spec{B}x{gamma}x{V}")
    if V > 1:
        assert 0 < n_o.mean() < gamma        # both outcomes occur: the test is not vacuous


def test_all_accepted_and_rejections_forced():
    """q = p accepts every drafted token (the bonus token comes from p_gamma); a drafted token the
    target gives probability 0 (logit -inf) is rejected; an out-of-vocabulary token is rejected."""
    log("case: spec accept forced outcomes")
    t, d, x, u = case(77, 8, 5, 512)
    d = t[:, :5].copy()
    u[:, :5] = np.minimum(u[:, :5], 0.999)
    n_o = compare(t, d, x, u, "spec-q=p")
    assert (n_o == 5).all()
    t2 = t.copy()
    t2[np.arange(8), 2, x[:, 2]] = -np.inf
    n_o = compare(t2, d, x, u, "spec-p=0")
    assert (n_o == 2).all()
    x3 = x.copy()
    x3[:, 1] = 512
    x3[0, 1] = -1
    n_g, _ = run_gpu(t, d, x3, u)
    assert (n_g == 1).all()
    # q = p and the least likely token drafted, with u_0 just below 1: p / (q + 1e-8) < u_0, so
    # it is rejected and the residual (p - q)_+ is exactly zero; the token comes from p_0
    x4 = x.copy()
    x4[:, 0] = t[:, 0].argmin(axis=-1)
    u4 = u.copy()
    u4[:, 0] = np.nextafter(np.float32(1), np.float32(0))
    n_o = compare(t, d, x4, u4, "spec-residual-0")
    assert (n_o == 0).all()


def test_first_token_follows_target_distribution_on_gpu():
    """20000 rounds (one launch) with the same logits and drafted tokens drawn from q: the first
    emitted token is distributed as p_0 (chi-square, df 15, p = 1e-4)."""
    log("case: spec accept first-token distribution")
    rng = np.random.default_rng(31)
    V, gamma, N = 16, 4, 20000
    t1 = rng.normal(0, 1.5, (gamma + 1, V)).astype(np.float32)
    d1 = (t1[:gamma] + rng.normal(0, 1.0, (gamma, V))).astype(np.float32)
    q = softmax(d1)
    x = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(gamma)], axis=1).astype(np.int32)
    u = rng.random((N, gamma + 1)).astype(np.float32)
    t = np.ascontiguousarray(np.broadcast_to(t1, (N, gamma + 1, V)))
    d = np.ascontiguousarray(np.broadcast_to(d1, (N, gamma, V)))
    n, nxt = run_gpu(t, d, x, u)
    first = np.where(n >= 1, x[:, 0], nxt)
    p0 = softmax(t1[0])
    obs = np.bincount(first, minlength=V)
    chi2 = float((((obs - N * p0) ** 2) / (N * p0)).sum())
    log(f"spec first-token chi2 {chi2:.1f} (df {V - 1}), rejection rate {float((n < gamma).mean()):.3f}")
    assert chi2 < 42.0, (chi2, obs, N * p0)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_match_oracle(seed):
    """Seeded random batch (1 .. 64), gamma (1 .. 15), vocabulary (log-uniform, 1 .. ~70000 or,
    for every other seed, 4097 .. ~70000: ragged in the 4096-token parts), logit spread and draft
    noise; decisions exact away from the oracle's 1e-5 margin, valid everywhere."""
    rng = np.random.default_rng(9000 + seed)
    B, gamma = int(rng.integers(1, 65)), int(rng.integers(1, 16))
    lo = 0.0 if seed % 2 else np.log(4097)          # half of the cases span several parts
    V = int(np.exp(rng.uniform(lo, np.log(70000))))
    spread, noise = float(rng.choice([2.0, 3.0, 4.0])), float(rng.choice([0.5, 1.0, 2.0]))
    log(f"case: spec accept random seed {seed}: B={B} gamma={gamma} V={V} spread={spread} "
        f"noise={noise}")
    t, d, x, u = case(9100 + seed, B, gamma, V, spread=spread, noise=noise)
    n_g, nxt_g = run_gpu(t, d, x, u)
    n_o, nxt_o, mg = oracle.spec_accept(t, d, x, u)
    close = mg < 1e-5
    bad = ~close & ((n_g != n_o) | (nxt_g != nxt_o))
    log(f"random{seed}: near-boundary {int(close.sum())} of {B}, mismatches {int(bad.sum())}")
    assert not bad.any(), (np.nonzero(bad)[0][:5], n_g[bad][:5], n_o[bad][:5])
    assert ((n_g >= 0) & (n_g <= gamma)).all() and ((nxt_g >= 0) & (nxt_g < V)).all()
