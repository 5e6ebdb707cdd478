"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every expectation comes from a closed form
(grid-exact groups, ties, constant groups), a bound the quantizer must satisfy, an identity of
the cache's bookkeeping, or an independent library routine (numpy's fp16 conversion, torch's
float64 scaled_dot_product_attention on the CPU).

Sources: QuantSpec Guide (aifetchly), quantizer listing and "Double Full-Precision Cache
Buffer"; Pith review of arXiv:2502.10424, "What carries the argument", Fig. 3, Fig. 7 and
reference [128].
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleCache, OracleError
from hierarchical_quantized_kv_amd import synth

G = 128


def setup_module(_):
    oracle.build(force=False)


# ------------------------------------------------------------------------------------------
# fp16
# ------------------------------------------------------------------------------------------

def test_half_to_float_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.lib().orc_half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ------------------------------------------------------------------------------------------
# Quantizer
# ------------------------------------------------------------------------------------------

def grid_group(rng, n, z0):
    """x = (k - z0) * 2^-5 with k in 0..255 and both 0 and 255 present: exact in fp16,
    so the quantizer must return s = 2^-5, z = z0 and codes k exactly."""
    k = rng.integers(0, 256, size=n)
    k[rng.choice(n, 2, replace=False)] = [0, 255]
    x = ((k - z0) * 2.0 ** -5).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), (k - z0) * 2.0 ** -5)
    return k, x


@pytest.mark.parametrize("n", [64, 128])
def test_grid_exact_group_roundtrips_exactly(n):
    rng = np.random.default_rng(1)
    for _ in range(200):
        z0 = int(rng.integers(0, 256))
        k, x = grid_group(rng, n, z0)
        s, z, c = oracle.quantize_group(x)
        assert s == 2.0 ** -5 and z == z0
        assert np.array_equal(c, k)
        # full dequantization is exact; the draft dequantization is the midpoint of the
        # upper nibble's 16-code bucket (off = 8) or its lower edge (off = 0)
        for i in range(0, n, 7):
            assert oracle.dequant_full(c[i], s, z) == float(x[i])
            cu = int(k[i]) >> 4
            assert oracle.dequant_upper(cu, s, z, 8) == (16 * cu + 8 - z0) * 2.0 ** -5
            assert oracle.dequant_upper(cu, s, z, 0) == (16 * cu - z0) * 2.0 ** -5


def test_round_half_to_even_on_exact_ties():
    """Values exactly halfway between two codes round to the even one, like torch.round."""
    z0 = 100
    for k in range(1, 255):
        x = np.array([(0 - z0) * 2.0 ** -5, (255 - z0) * 2.0 ** -5, (k + 0.5 - z0) * 2.0 ** -5],
                     dtype=np.float16)
        s, z, c = oracle.quantize_group(x)
        assert s == 2.0 ** -5 and z == z0
        t = k + 0.5 - z0                      # exact x / s: a tie
        assert c[2] == round(t) + z0          # Python's round() is half-to-even
        assert c[2] % 2 == (z0 % 2)           # the rounded quotient is even


def test_constant_group_clamps_scale():
    for v in (0.0, 0.5, -3.25, 1000.0):
        x = np.full(128, v, dtype=np.float16)
        s, z, c = oracle.quantize_group(x)
        assert s == np.float32(1e-8)
        assert np.all(c == 0)
        assert abs(oracle.dequant_full(0, s, z) - v) <= abs(v) * 2.0 ** -20 + 1e-12


def random_groups(rng, n_groups, n):
    for i in range(n_groups):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(n)
        elif kind == 1:
            x = rng.standard_normal(n) * 8.0 + rng.standard_normal()
        elif kind == 2:
            z = rng.standard_normal(n)
            x = z / np.sqrt((rng.standard_normal((3, n)) ** 2).sum(0) / 3)
        else:
            x = rng.uniform(0.5, 2.0, n)      # all-positive group: zero-point below 0
        yield x.astype(np.float16)


@pytest.mark.parametrize("n", [64, 128])
def test_code_range_and_roundtrip_bounds(n):
    """code(min) = 0, code(max) in {254, 255}; |x - xhat| <= s/2 (plus the fp32 division
    slack); draft error <= 8.5 s (off = 8) or 15.5 s (off = 0), under one upper step 16 s."""
    rng = np.random.default_rng(2)
    slack = 2.0 ** -14
    for x in random_groups(rng, 400, n):
        s, z, c = oracle.quantize_group(x)
        xf = x.astype(np.float64)
        assert s > 1e-8
        assert c[np.argmin(xf)] == 0
        assert c[np.argmax(xf)] in (254, 255)
        full = np.array([oracle.dequant_full(ci, s, z) for ci in c])
        assert np.max(np.abs(full - xf)) <= (0.5 + slack) * s
        for off, bound in ((8, 8.5), (0, 15.5)):
            up = np.array([oracle.dequant_upper(ci >> 4, s, z, off) for ci in c])
            assert np.max(np.abs(up - xf)) <= (bound + slack) * s < 16 * s


# ------------------------------------------------------------------------------------------
# Attention: reference computations with torch float64 SDPA on the CPU
# ------------------------------------------------------------------------------------------

def sdpa(q, k, v, mask=None, scale=1.0):
    """q [m][D], k/v [n][D] (float64) -> [m][D] via torch's CPU float64 SDPA."""
    qt = torch.as_tensor(np.asarray(q, np.float64))[None, None]
    kt = torch.as_tensor(np.asarray(k, np.float64))[None, None]
    vt = torch.as_tensor(np.asarray(v, np.float64))[None, None]
    mt = None if mask is None else torch.as_tensor(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt,
                                                            scale=scale)[0, 0].numpy()


def f64(a):
    return np.asarray(a, np.float16).astype(np.float64)


@pytest.mark.parametrize("D", [64, 128])
def test_tail_only_attention_matches_sdpa(D):
    """nq = 0: draft is plain softmax attention over the fp16 tail; verify is the same with the
    causal mask of the last m tokens."""
    B, H, n = 2, 3, 150
    k, v = synth.kv_host(B, n, H, D, 11, 12)
    c = OracleCache(1, B, H, D, G, 4 * G, 6)
    c.append(0, k, v)
    q = synth.queries_host(B, None, H, D, 13)
    out = c.attend_draft(0, q, sm_scale=0.7)
    for b in range(B):
        for h in range(H):
            ref = sdpa(f64(q[b, h])[None], f64(k[b, :, h]), f64(v[b, :, h]), scale=0.7)[0]
            assert np.max(np.abs(out[b, h] - ref)) < 1e-6
    m = 7
    qv = synth.queries_host(B, m, H, D, 14)
    outv = c.attend_verify(0, qv, sm_scale=1.3)
    mask = np.zeros((m, n), dtype=bool)
    for i in range(m):
        mask[i, : n - m + i + 1] = True
    for b in range(B):
        for h in range(H):
            ref = sdpa(f64(qv[b, :, h]), f64(k[b, :, h]), f64(v[b, :, h]), mask, scale=1.3)
            assert np.max(np.abs(outv[b, :, h] - ref)) < 1e-6


def grid_kv(rng, n_groups, H, D):
    """Keys and values [1][n][H][D] whose every quantization group is grid-exact: keys per
    (head, channel) over each G-token group, values per (token, head) over D channels."""
    n = n_groups * G
    kk = np.zeros((n, H, D), np.int64)
    vk = np.zeros((n, H, D), np.int64)
    kz = rng.integers(0, 256, size=(n_groups, H, D))
    vz = rng.integers(0, 256, size=(n, H))
    for g in range(n_groups):
        blk = rng.integers(0, 256, size=(G, H, D))
        blk[0], blk[1] = 0, 255
        kk[g * G:(g + 1) * G] = blk
    vk[:] = rng.integers(0, 256, size=(n, H, D))
    vk[:, :, 0], vk[:, :, 1] = 0, 255
    kx = (kk - np.repeat(kz, G, axis=0)) * 2.0 ** -5
    vx = (vk - vz[:, :, None]) * 2.0 ** -5
    return (kk, kz, kx.astype(np.float16)[None], vk, vz, vx.astype(np.float16)[None])


def test_grid_exact_cache_verify_equals_unquantized_and_draft_equals_upper_formula():
    """On a grid-exact cache the verify dequantization is lossless, so verify attention equals
    plain attention over the original fp16 keys/values; the draft attention equals plain
    attention over (16 * (k >> 4) + 8 - z0) * 2^-5 built here from the integer grid."""
    rng = np.random.default_rng(3)
    H, D, ng = 2, 64, 3
    kk, kz, kx, vk, vz, vx = grid_kv(rng, ng, H, D)
    c = OracleCache(1, 1, H, D, G, 4 * G, 4)
    for g in range(ng):
        c.append(0, kx[:, g * G:(g + 1) * G], vx[:, g * G:(g + 1) * G])
        assert c.flush(0)[0] == 1
    tk, tv = synth.kv_host(1, 40, H, D, 21, 22)
    c.append(0, tk, tv)
    nq, nt, head = c.state(0)
    assert (nq[0], nt[0]) == (ng * G, 40)
    for h in range(H):
        assert np.array_equal(c.codes(0, 0, h)[: ng * G], kk[:, h])
        assert np.array_equal(c.codes(0, 0, h, which_v=True)[: ng * G], vk[:, h])
    q = synth.queries_host(1, None, H, D, 23, gain=3.0)
    draft = c.attend_draft(0, q)
    m = 5
    qv = synth.queries_host(1, m, H, D, 24)
    ver = c.attend_verify(0, qv)
    kz_tok = np.repeat(kz, G, axis=0)
    for h in range(H):
        kall = np.concatenate([f64(kx[0, :, h]), f64(tk[0, :, h])])
        vall = np.concatenate([f64(vx[0, :, h]), f64(tv[0, :, h])])
        mask = np.zeros((m, len(kall)), bool)
        for i in range(m):
            mask[i, : ng * G + 40 - m + i + 1] = True
        ref = sdpa(f64(qv[0, :, h]), kall, vall, mask)
        assert np.max(np.abs(ver[0, :, h] - ref)) < 1e-6
        ku = (16 * (kk[:, h] >> 4) + 8 - kz_tok[:, h]) * 2.0 ** -5
        vu = (16 * (vk[:, h] >> 4) + 8 - vz[:, h][:, None]) * 2.0 ** -5
        refd = sdpa(f64(q[0, h])[None], np.concatenate([ku, f64(tk[0, :, h])]),
                    np.concatenate([vu, f64(tv[0, :, h])]))[0]
        assert np.max(np.abs(draft[0, h] - refd)) < 1e-6


@pytest.mark.parametrize("off,nibble,m16", [(8, 8, False), (0, 0, False), (8, 8, True),
                                            (0, 0, True)])
def test_draft_equals_verify_when_every_lower_nibble_is_the_draft_offset(off, nibble, m16):
    """The draft reconstruction (16 C_U + off - z) s is the full one (C8 - z) s of a code whose
    lower nibble is off (with fp16 metadata: s (16 C_U + off) + b and s C8 + b): after setting
    every stored lower nibble to off, a one-query verify (which sees the whole tail) equals the
    draft, exactly.  A wrong shift, nibble or offset in either dequantization fails it."""
    H, D = 3, 64
    c = OracleCache(1, 2, H, D, G, 4 * G, 4, draft_offset=off, meta_fp16=m16)
    k, v = synth.kv_host(2, 2 * G + 50, H, D, 41, 42)
    c.prefill(0, k, v, n=[2 * G + 50, G + 7])
    q = synth.queries_host(2, None, H, D, 43, gain=2.0)
    before = c.attend_draft(0, q)
    c.set_lower_nibbles(0, nibble)
    draft = c.attend_draft(0, q)
    ver = c.attend_verify(0, q[:, None])[:, 0]
    assert np.array_equal(draft, before)            # the draft never reads the lower nibbles
    assert np.array_equal(draft, ver)
    c.set_lower_nibbles(0, nibble ^ 1)              # any other nibble breaks the identity
    assert not np.array_equal(c.attend_verify(0, q[:, None])[:, 0], draft)


def test_single_token_and_zero_query_closed_forms():
    rng = np.random.default_rng(4)
    H, D = 2, 64
    k, v = synth.kv_host(1, 1, H, D, 31, 32)
    c = OracleCache(1, 1, H, D, G, 2 * G, 4)
    c.append(0, k, v)
    out = c.attend_draft(0, synth.queries_host(1, None, H, D, 33))
    assert np.array_equal(out[0], v[0, 0].astype(np.float32))      # one key: out = v
    # q = 0: uniform softmax, out = mean of every dequantized value (exact on a grid cache)
    kk, kz, kx, vk, vz, vx = grid_kv(rng, 2, H, D)
    c2 = OracleCache(1, 1, H, D, G, 2 * G, 4)
    for g in range(2):
        c2.append(0, kx[:, g * G:(g + 1) * G], vx[:, g * G:(g + 1) * G])
        c2.flush(0)
    tk, tv = synth.kv_host(1, 10, H, D, 34, 35)
    c2.append(0, tk, tv)
    out = c2.attend_verify(0, np.zeros((1, 1, H, D), np.float16))
    ref = np.concatenate([f64(vx[0]), f64(tv[0])]).mean(axis=0)
    assert np.max(np.abs(out[0, 0] - ref)) < 1e-6


def test_attention_over_explicit_dequantized_cache():
    """Random (not grid) cache: the oracle's attention equals SDPA over keys/values
    dequantized here from the read-back codes and metadata, with the tail appended in
    logical order (checks the token bookkeeping, group indexing and tail ordering)."""
    B, H, D = 2, 2, 64
    c = OracleCache(1, B, H, D, G, 4 * G, 6)
    k, v = synth.kv_host(B, 2 * G, H, D, 41, 42, outliers=synth.outlier_channels(H, D, 43))
    c.append(0, k[:, :G], v[:, :G])
    c.flush(0)
    c.append(0, k[:, G:], v[:, G:])
    c.rollback(0, [5, 0])
    c.flush(0, min_tail=G)                 # b=0 has 123 < G tail tokens: only b=1 flushes
    k2, v2 = synth.kv_host(B, 9, H, D, 44, 45)
    c.append(0, k2, v2, n=[9, 4])
    nq, nt, head = c.state(0)
    assert list(nq) == [G, 2 * G] and list(nt) == [G - 5 + 9, 4] and list(head) == [G, 0]
    q = synth.queries_host(B, None, H, D, 46)
    out = c.attend_draft(0, q, sm_scale=1.1)
    m = 3
    qv = synth.queries_host(B, m, H, D, 47)
    outv = c.attend_verify(0, qv)
    for b in range(B):
        logical = [k[b, G:2 * G - 5]] if b == 0 else []
        vlog = [v[b, G:2 * G - 5]] if b == 0 else []
        n2 = 9 if b == 0 else 4
        tk = np.concatenate(logical + [k2[b, :n2]]) if logical else k2[b, :n2]
        tvv = np.concatenate(vlog + [v2[b, :n2]]) if vlog else v2[b, :n2]
        for h in range(H):
            codes_k = c.codes(0, b, h)[: nq[b]].astype(np.float64)
            codes_v = c.codes(0, b, h, True)[: nq[b]].astype(np.float64)
            km, vm = c.meta(0, b, h)
            ks = np.repeat(km[:, :, 0], G, axis=0)[: nq[b]].astype(np.float64)
            kz = np.repeat(km[:, :, 1], G, axis=0)[: nq[b]].astype(np.float64)
            vs = vm[: nq[b], 0:1].astype(np.float64)
            vz = vm[: nq[b], 1:2].astype(np.float64)
            kf, vf = (codes_k - kz) * ks, (codes_v - vz) * vs
            ku = (16 * np.floor(codes_k / 16) + 8 - kz) * ks
            vu = (16 * np.floor(codes_v / 16) + 8 - vz) * vs
            ka = np.concatenate([ku, f64(tk[:, h])])
            va = np.concatenate([vu, f64(tvv[:, h])])
            ref = sdpa(f64(q[b, h])[None], ka, va, scale=1.1)[0]
            assert np.max(np.abs(out[b, h] - ref)) < 1e-6
            ka = np.concatenate([kf, f64(tk[:, h])])
            va = np.concatenate([vf, f64(tvv[:, h])])
            n = len(ka)
            mask = np.zeros((m, n), bool)
            for i in range(m):
                mask[i, : n - m + i + 1] = True
            ref = sdpa(f64(qv[b, :, h]), ka, va, mask)
            assert np.max(np.abs(outv[b, :, h] - ref)) < 1e-6


# ------------------------------------------------------------------------------------------
# State machine
# ------------------------------------------------------------------------------------------

def test_append_rollback_append_is_identity():
    B, H, D = 2, 2, 64
    k, v = synth.kv_host(B, 20, H, D, 51, 52)
    a = OracleCache(1, B, H, D, G, 2 * G, 4)
    b = OracleCache(1, B, H, D, G, 2 * G, 4)
    a.append(0, k[:, :10], v[:, :10])
    b.append(0, k[:, :10], v[:, :10])
    junk_k, junk_v = synth.kv_host(B, 4, H, D, 53, 54)
    a.append(0, junk_k, junk_v)
    a.rollback(0, [4, 4])
    a.append(0, k[:, 10:], v[:, 10:])
    b.append(0, k[:, 10:], v[:, 10:])
    for x, y in zip(a.state(0), b.state(0)):
        assert np.array_equal(x, y)
    q = synth.queries_host(B, None, H, D, 55)
    assert np.array_equal(a.attend_draft(0, q), b.attend_draft(0, q))


def test_quantized_tier_is_a_function_of_the_committed_stream():
    """A speculative trace (draft appends, rollbacks, verify appends, acceptance, flushes)
    leaves exactly the codes and metadata of a fresh prefill of the committed tokens."""
    B, H, D, gamma = 1, 2, 64, 4
    rng = np.random.default_rng(6)
    trace = OracleCache(1, B, H, D, G, 6 * G, gamma)
    committed_k, committed_v = [], []
    base_k, base_v = synth.kv_host(B, 60, H, D, 61, 62)
    trace.append(0, base_k, base_v)
    committed_k.append(base_k)
    committed_v.append(base_v)
    rnd = 0
    while trace.state(0)[0][0] < 3 * G:
        for _ in range(gamma):                      # draft K/V, discarded before verify
            dk, dv = synth.kv_host(B, 1, H, D, 1000 + rnd * 10, 2000 + rnd * 10)
            trace.append(0, dk, dv)
        trace.rollback(0, [gamma])
        tk, tv = synth.kv_host(B, gamma + 1, H, D, 3000 + rnd, 4000 + rnd)
        trace.append(0, tk, tv)
        a = synth.acceptance(rng, gamma)
        trace.rollback(0, [gamma - a])
        committed_k.append(tk[:, : a + 1])
        committed_v.append(tv[:, : a + 1])
        trace.flush(0, G)
        rnd += 1
    ck = np.concatenate(committed_k, axis=1)
    cv = np.concatenate(committed_v, axis=1)
    fresh = OracleCache(1, B, H, D, G, 6 * G, gamma)
    pos = 0
    while ck.shape[1] - pos >= G:
        fresh.append(0, ck[:, pos:pos + G], cv[:, pos:pos + G])
        fresh.flush(0)
        pos += G
    fresh.append(0, ck[:, pos:], cv[:, pos:])
    nq = trace.state(0)[0][0]
    assert fresh.state(0)[0][0] == nq and trace.state(0)[1][0] == fresh.state(0)[1][0]
    for h in range(H):
        for which in (False, True):
            assert np.array_equal(trace.codes(0, 0, h, which), fresh.codes(0, 0, h, which))
        for x, y in zip(trace.meta(0, 0, h), fresh.meta(0, 0, h)):
            assert np.array_equal(x, y)


def test_prefill_equals_group_by_group_append_and_flush():
    """Quantize once: a prompt whose whole groups pass through the buffer and are quantized as
    they leave it, the rest left there -- the same counters, codes, metadata and live tail as
    append(G) + flush per group followed by an append of the rest, for ragged prompts and after
    an earlier group."""
    B, H, D = 4, 2, 64
    lens = [0, G - 1, 3 * G, 2 * G + 77]
    k, v = synth.kv_host(B, max(lens), H, D, 95, 96)
    k0, v0 = synth.kv_host(B, G, H, D, 97, 98)
    a = OracleCache(1, B, H, D, G, 6 * G, 4)
    ref = OracleCache(1, B, H, D, G, 6 * G, 4)
    for c in (a, ref):                               # one earlier group on sequence 3
        c.append(0, k0, v0, n=[0, 0, 0, G])
        c.flush(0)
    a.prefill(0, k, v, lens)
    n_groups = max(L // G for L in lens)
    for g in range(n_groups):
        n = [G if L >= (g + 1) * G else 0 for L in lens]
        ref.append(0, k[:, g * G:(g + 1) * G], v[:, g * G:(g + 1) * G], n=n)
        ref.flush(0)
    rest = [L - (L // G) * G for L in lens]
    rk = np.zeros((B, G, H, D), np.float16)
    rv = np.zeros((B, G, H, D), np.float16)
    for b, L in enumerate(lens):
        rk[b, : rest[b]] = k[b, L - rest[b]: L]
        rv[b, : rest[b]] = v[b, L - rest[b]: L]
    ref.append(0, rk, rv, n=rest)
    for x, y in zip(a.state(0), ref.state(0)):
        assert np.array_equal(x, y)
    nq, nt, head = a.state(0)
    assert list(nq) == [0, 0, 3 * G, 3 * G] and list(nt) == [0, G - 1, 0, 77]
    assert list(head) == [0, 0, G, G]                # one toggle per quantized group
    ia, ir = a.export_layer(0), ref.export_layer(0)
    for name in ("uk", "lk", "uv", "lv", "kmeta", "vmeta"):
        assert np.array_equal(ia[name], ir[name]), name
    for b in range(B):
        slots = [(int(head[b]) + i) % (2 * G) for i in range(int(nt[b]))]
        assert np.array_equal(ia["tail_k"][b][:, slots], ir["tail_k"][b][:, slots])
        assert np.array_equal(ia["tail_v"][b][:, slots], ir["tail_v"][b][:, slots])


def test_prefill_errors_leave_state_unchanged():
    H, D = 1, 64
    k, v = synth.kv_host(2, 3 * G, H, D, 101, 102)
    c = OracleCache(1, 2, H, D, G, 2 * G, 4)
    c.append(0, k[:, :5], v[:, :5], n=[5, 0])
    with pytest.raises(OracleError) as e:
        c.prefill(0, k, v, [G, G])                   # sequence 0 has a non-empty tail
    assert e.value.code == 3
    with pytest.raises(OracleError) as e:
        c.prefill(0, k, v, [0, 3 * G])               # 3 groups > capacity of 2
    assert e.value.code == 2
    with pytest.raises(OracleError) as e:
        c.prefill(0, k[:, :G], v[:, :G], [0, G + 1])  # n > n_max
    assert e.value.code == 1
    assert [list(x) for x in c.state(0)] == [[0, 0], [5, 0], [0, 0]]
    c.prefill(0, k, v, [0, 2 * G + 9])               # the empty sequence may take a prompt
    assert [list(x) for x in c.state(0)] == [[0, 2 * G], [5, 9], [0, 0]]


def test_ring_head_toggles_and_logical_order_survives_flush():
    H, D = 1, 64
    k, v = synth.kv_host(1, 3 * G, H, D, 71, 72)
    c = OracleCache(1, 1, H, D, G, 4 * G, 4)
    c.append(0, k[:, : G + 30], v[:, : G + 30])
    assert list(c.state(0)[2]) == [0]
    c.flush(0)
    assert [x[0] for x in c.state(0)] == [G, 30, G]
    c.append(0, k[:, G + 30: 2 * G + 50], v[:, G + 30: 2 * G + 50])
    c.flush(0)
    assert [x[0] for x in c.state(0)] == [2 * G, 50, 0]
    # the remaining tail is tokens 2G .. 2G+49, attended as such
    q = synth.queries_host(1, None, H, D, 73)
    ref_c = OracleCache(1, 1, H, D, G, 4 * G, 4)
    ref_c.append(0, k[:, : G], v[:, : G]); ref_c.flush(0)
    ref_c.append(0, k[:, G: 2 * G], v[:, G: 2 * G]); ref_c.flush(0)
    ref_c.append(0, k[:, 2 * G: 2 * G + 50], v[:, 2 * G: 2 * G + 50])
    assert np.array_equal(c.attend_draft(0, q), ref_c.attend_draft(0, q))


def test_error_paths_leave_state_unchanged():
    H, D = 1, 64
    k, v = synth.kv_host(1, 2 * G + 1, H, D, 81, 82)
    c = OracleCache(1, 2, H, D, G, G, 4)
    k2 = np.concatenate([k, k]); v2 = np.concatenate([v, v])
    with pytest.raises(OracleError) as e:
        c.append(0, k2, v2)                          # 2G + 1 > ring
    assert e.value.code == 2
    c.append(0, k2[:, :10], v2[:, :10], n=[10, 3])
    with pytest.raises(OracleError) as e:
        c.rollback(0, [2, 4])                        # 4 > nt of b = 1
    assert e.value.code == 3
    assert list(c.state(0)[1]) == [10, 3]
    with pytest.raises(OracleError) as e:
        c.attend_verify(0, np.zeros((2, 4, H, D), np.float16))  # m = 4 > nt = 3
    assert e.value.code == 3
    c.append(0, k2[:, :G], v2[:, :G])
    c.flush(0)                                       # both reach nq = G = capacity
    c.append(0, k2[:, :G], v2[:, :G], n=[G, 0])
    with pytest.raises(OracleError) as e:
        c.flush(0)                                   # b = 0 would exceed max_ctx
    assert e.value.code == 2
    assert list(c.state(0)[0]) == [G, G] and list(c.state(0)[1]) == [10 + G, 3]
    empty = OracleCache(1, 1, H, D, G, G, 4)
    with pytest.raises(OracleError) as e:
        empty.attend_draft(0, np.zeros((1, H, D), np.float16))
    assert e.value.code == 3


def test_layout_export_matches_split_identity():
    """Every packed nibble pair of the exported arena image satisfies C8 = 16 C_U + C_L against
    the logical codes, at the byte positions the layout defines."""
    B, H, D = 1, 2, 64
    c = OracleCache(1, B, H, D, G, 2 * G, 4)
    k, v = synth.kv_host(B, 2 * G, H, D, 91, 92)
    for g in range(2):
        c.append(0, k[:, g * G:(g + 1) * G], v[:, g * G:(g + 1) * G])
        c.flush(0)
    img = c.export_layer(0)
    for h in range(H):
        ck = c.codes(0, 0, h).astype(np.int64)
        cv = c.codes(0, 0, h, True).astype(np.int64)
        uk, lk = img["uk"][0, h].astype(np.int64), img["lk"][0, h].astype(np.int64)
        even = 16 * (uk & 15) + (lk & 15)
        odd = 16 * (uk >> 4) + (lk >> 4)
        assert np.array_equal(even, ck[:, 0::2]) and np.array_equal(odd, ck[:, 1::2])
        uv, lv = img["uv"][0, h].astype(np.int64), img["lv"][0, h].astype(np.int64)
        for g in range(2):
            for e in range(2):                          # two halves of G/2 tokens
                tok = cv[g * G + e * G // 2: g * G + (e + 1) * G // 2]   # [G/2][D]
                ev = 16 * (uv[g, e] & 15) + (lv[g, e] & 15)   # [D][G/4]: tokens 0, 2, 4, ...
                od = 16 * (uv[g, e] >> 4) + (lv[g, e] >> 4)
                assert np.array_equal(ev, tok[0::2].T) and np.array_equal(od, tok[1::2].T)
        km, vm = c.meta(0, 0, h)
        assert np.array_equal(img["kmeta"][0, h], km) and np.array_equal(img["vmeta"][0, h], vm)


# ------------------------------------------------------------------------------------------
# Speculative accept / correct
# ------------------------------------------------------------------------------------------

def _softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_spec_accept_first_token_follows_the_target_distribution():
    """The point of the correction step: whatever the draft distribution, the first token the
    round emits (x_0 if accepted, else the resampled one) is distributed as p_0.  30000 rounds
    with fixed logits, drafted tokens drawn from q_i, fresh uniforms; chi-square against p_0."""
    rng = np.random.default_rng(2024)
    V, gamma, N = 6, 3, 30000
    t = rng.normal(0, 1.5, (gamma + 1, V)).astype(np.float32)
    d = (t[:gamma] + rng.normal(0, 1.0, (gamma, V))).astype(np.float32)
    q = _softmax(d)
    x = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(gamma)], axis=1).astype(np.int32)
    u = rng.random((N, gamma + 1)).astype(np.float32)
    n, nxt, _ = oracle.spec_accept(np.broadcast_to(t, (N, gamma + 1, V)),
                                   np.broadcast_to(d, (N, gamma, V)), x, u)
    first = np.where(n >= 1, x[:, 0], nxt)
    p0 = _softmax(t[0])
    obs = np.bincount(first, minlength=V)
    chi2 = float((((obs - N * p0) ** 2) / (N * p0)).sum())
    assert chi2 < 25.7, (chi2, obs, N * p0)     # df 5, p = 1e-4
    # and the draft is not the target: some rounds reject (the test is not vacuous)
    assert 0.05 < float((n < gamma).mean()) < 0.95


def test_spec_accept_closed_forms():
    ninf = -np.inf
    # p_0 = (1/2, 1/2, 0, 0), q_0 = (0, 1, 0, 0), drafted token 1: accepted iff
    # u_0 <= 1/2 / (1 + 1e-8), just below 1/2; the residual (p_0 - q_0)_+ = (1/2, 0, 0, 0) gives
    # token 0 whatever u_1; after an acceptance the sample comes from p_1 = (0, 0, 1, 0)
    t = np.array([[[0, 0, ninf, ninf], [ninf, ninf, 0, ninf]]], np.float32)
    d = np.array([[[ninf, 0, ninf, ninf]]], np.float32)
    for u0, u1, n_exp, tok_exp in ((0.7, 0.99, 0, 0), (0.7, 0.0, 0, 0), (0.3, 0.5, 1, 2),
                                   (0.5, 0.2, 0, 0), (0.4999, 0.2, 1, 2)):
        n, nxt, _ = oracle.spec_accept(t, d, np.array([[1]], np.int32),
                                       np.array([[u0, u1]], np.float32))
        assert (n[0], nxt[0]) == (n_exp, tok_exp), (u0, u1, n[0], nxt[0])
    # q = p: every test passes (u < 1 - 1e-6), then the inverse CDF of p_gamma
    rng = np.random.default_rng(5)
    V, gamma = 7, 4
    t = rng.normal(0, 1, (1, gamma + 1, V)).astype(np.float32)
    d = t[:, :gamma].copy()
    x = rng.integers(0, V, (1, gamma)).astype(np.int32)
    cdf = np.cumsum(_softmax(t[0, gamma]))
    for ug in (0.0, 0.3, 0.8, 0.999):
        n, nxt, _ = oracle.spec_accept(t, d, x, np.array([[0.5] * gamma + [ug]], np.float32))
        assert n[0] == gamma
        assert nxt[0] == int(np.searchsorted(cdf, np.float32(ug) * cdf[-1], side="right"))
    # a drafted token outside the vocabulary is rejected at its position
    x2 = x.copy()
    x2[0, 2] = V
    n, _, _ = oracle.spec_accept(t, d, x2, np.array([[0.5] * gamma + [0.1]], np.float32))
    assert n[0] == 2


# ------------------------------------------------------------------------------------------
# fp16 metadata (scale s, offset b = -s z)
# ------------------------------------------------------------------------------------------

def np_half_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_float_to_half_matches_numpy():
    """Round to nearest even against numpy's fp32 -> fp16 conversion: every finite half, the
    midpoints between neighbours (exact ties), points just off them, subnormals, overflow."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = h[np.isfinite(h)].astype(np.float64)
    pos = np.unique(np.abs(fin))
    mids = (pos[:-1] + pos[1:]) / 2                       # exact in fp32 (12 significant bits)
    xs = [fin, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
          np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.random.default_rng(7).standard_normal(20000) * 10.0 ** np.random.default_rng(8).uniform(-9, 5, 20000),
          np.array([65504.0, 65519.0, 65520.0, 7e4, -7e4, 1e-8, 2.9e-8, 3.0e-8, 2.0 ** -25, 2.0 ** -24])]
    x = np.concatenate([np.asarray(a, np.float64) for a in xs]).astype(np.float32)
    got = np.array([oracle.float_to_half(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, np_half_bits(x))


def _pair_caches(rng_seed, H=3, D=64, groups=3, m16_only=False):
    k, v = synth.kv_host(1, groups * G, H, D, rng_seed, rng_seed + 1,
                         outliers=synth.outlier_channels(H, D, rng_seed + 2))
    caches = []
    for m16 in (False, True):
        c = OracleCache(1, 1, H, D, G, groups * G, 4, meta_fp16=m16)
        c.prefill(0, k, v)
        caches.append(c)
    return k, v, caches


def test_meta16_pairs_are_the_fp16_values_of_scale_and_offset():
    """Same input, both formats: identical codes; the fp16 pairs are numpy's fp16 of the fp32
    cache's s and of -(s z) (fp32 product, clamped to +-65504)."""
    H, D = 3, 64
    _, _, (c32, c16) = _pair_caches(51, H, D)
    for h in range(H):
        for which in (False, True):
            assert np.array_equal(c32.codes(0, 0, h, which), c16.codes(0, 0, h, which))
        for m32, m16 in zip(c32.meta(0, 0, h), c16.meta(0, 0, h)):
            s, z = m32[..., 0], m32[..., 1]
            b = np.clip(-(s * z), np.float32(-65504), np.float32(65504))
            assert b.dtype == np.float32
            assert np.array_equal(m16[..., 0], s.astype(np.float16).astype(np.float32))
            assert np.array_equal(m16[..., 1], b.astype(np.float16).astype(np.float32))


def test_meta16_dequantization_within_rounding_bound():
    """|(s C + b)_fp16 - (C - z) s| <= C |s16 - s| + |b16 - b| + |b - (-s z)| with each fp16
    rounding at most half an ulp (2^-11 relative, 2^-25 absolute below the normal range) and
    the fp32 product at most 2^-24 relative."""
    H, D = 3, 64
    _, _, (c32, c16) = _pair_caches(61, H, D)
    for h in range(H):
        for which in (False, True):
            codes = c32.codes(0, 0, h, which).astype(np.float64)
            (km32, vm32), (km16, vm16) = c32.meta(0, 0, h), c16.meta(0, 0, h)
            m32, m16 = (vm32, vm16) if which else (km32, km16)
            if which:
                s, z = m32[:, 0:1], m32[:, 1:2]
                s16, b16 = m16[:, 0:1], m16[:, 1:2]
            else:
                s, z = (np.repeat(m32[:, :, i], G, axis=0) for i in (0, 1))
                s16, b16 = (np.repeat(m16[:, :, i], G, axis=0) for i in (0, 1))
            s, z, s16, b16 = (a.astype(np.float64) for a in (s, z, s16, b16))
            x32 = (codes - z) * s
            x16 = s16 * codes + b16
            for up in (False, True):
                cc = 16 * np.floor(codes / 16) + 8 if up else codes
                x32 = (cc - z) * s
                x16 = s16 * cc + b16
                b = np.abs(s * z)
                bound = (cc * np.maximum(s * 2.0 ** -11, 2.0 ** -25) +
                         np.maximum(b * 2.0 ** -11, 2.0 ** -25) + b * 2.0 ** -23)
                assert np.all(np.abs(x16 - x32) <= bound)
                assert oracle.dequant16_full(int(codes[0, 0]), s16[0, 0], b16[0, 0]) == \
                    s16[0, 0] * codes[0, 0] + b16[0, 0]


@pytest.mark.parametrize("val", [0.0, 1.0, -3.5, 1000.0, -65504.0, 6.0e-8, 0.0999])
def test_meta16_constant_group_is_exact(val):
    """A constant group has s clamped to 1e-8 (fp16: 0) and every code 0 (the value sits at
    -z s): b is the value itself, so fp16 metadata reconstructs it exactly, both passes."""
    H, D = 1, 64
    x = np.full((1, G + 1, H, D), val, np.float16)   # one group and one tail token
    c = OracleCache(1, 1, H, D, G, 2 * G, 4, meta_fp16=True)
    c.prefill(0, x, x)
    km, vm = c.meta(0, 0, 0)
    km, vm = km[:1], vm[:G]                          # the quantized group
    assert np.all(km[..., 0] == 0) and np.all(vm[:, 0] == 0)
    assert np.all(km[..., 1] == np.float32(x[0, 0, 0, 0])) and np.all(vm[:, 1] == km[0, 0, 1])
    q = synth.queries_host(1, None, H, D, 71)
    ref = np.full(D, float(x[0, 0, 0, 0]), np.float32)
    assert np.array_equal(c.attend_draft(0, q)[0, 0], ref)
    assert np.array_equal(c.attend_verify(0, q[:, None])[0, 0, 0], ref)


def test_meta16_attention_over_explicit_dequantized_cache():
    """The oracle's attention with fp16 metadata equals SDPA over keys / values dequantized here
    as s C + b (draft: s (16 floor(C / 16) + 8) + b) from the read-back codes and pairs."""
    B, H, D = 1, 2, 64
    k, v = synth.kv_host(B, 2 * G + 30, H, D, 81, 82, outliers=synth.outlier_channels(H, D, 83))
    c = OracleCache(1, B, H, D, G, 4 * G, 6, meta_fp16=True)
    c.prefill(0, k, v)
    nq = 2 * G
    q = synth.queries_host(B, None, H, D, 84)
    m = 3
    qv = synth.queries_host(B, m, H, D, 85)
    out, outv = c.attend_draft(0, q, sm_scale=0.9), c.attend_verify(0, qv)
    for h in range(H):
        ck = c.codes(0, 0, h)[:nq].astype(np.float64)
        cv = c.codes(0, 0, h, True)[:nq].astype(np.float64)
        km, vm = c.meta(0, 0, h)
        ks, kb = (np.repeat(km[:, :, i], G, axis=0)[:nq].astype(np.float64) for i in (0, 1))
        vs, vb = vm[:nq, 0:1].astype(np.float64), vm[:nq, 1:2].astype(np.float64)
        tk, tv = f64(k[0, nq:, h]), f64(v[0, nq:, h])
        ku = ks * (16 * np.floor(ck / 16) + 8) + kb
        vu = vs * (16 * np.floor(cv / 16) + 8) + vb
        ref = sdpa(f64(q[0, h])[None], np.concatenate([ku, tk]), np.concatenate([vu, tv]),
                   scale=0.9)[0]
        assert np.max(np.abs(out[0, h] - ref)) < 1e-6
        ka, va = np.concatenate([ks * ck + kb, tk]), np.concatenate([vs * cv + vb, tv])
        n = len(ka)
        mask = np.zeros((m, n), bool)
        for i in range(m):
            mask[i, : n - m + i + 1] = True
        ref = sdpa(f64(qv[0, :, h]), ka, va, mask)
        assert np.max(np.abs(outv[0, :, h] - ref)) < 1e-6


# ------------------------------------------------------------------------------------------
# Top-k-bit draft from the same 8-bit code (Pith review, "Editorial extensions", "Reading
# between the lines"): the top k bits for the draft, all 8 for the verifier
# ------------------------------------------------------------------------------------------

def test_topk_dequant_reduces_to_the_4_bit_draft_and_to_verify():
    """k = 4 is the upper-plane draft and k = 8 the verify dequantization, exactly, for every
    code and both draft offsets, in both metadata formats."""
    rng = np.random.default_rng(61)
    for s, z in [(0.0123, 37.0), (1e-8, -5.0e7), (0.75, 255.0), (3.1, -12.0)]:
        s = float(np.float32(s))
        for off in (0, 8):
            for c8 in range(256):
                assert oracle.dequant_topk(c8, s, z, 4, off) == oracle.dequant_upper(c8 >> 4, s, z, off)
                assert oracle.dequant_topk(c8, s, z, 8, off) == oracle.dequant_full(c8, s, z)
                b = float(rng.standard_normal())
                assert oracle.dequant16_topk(c8, s, b, 4, off) == oracle.dequant16_upper(c8 >> 4, s, b, off)
                assert oracle.dequant16_topk(c8, s, b, 8, off) == oracle.dequant16_full(c8, s, b)


@pytest.mark.parametrize("n", [64, 128])
def test_topk_roundtrip_bounds(n):
    """|x - x^k| <= (2^(7-k) + 1/2 + 2^-14) s with the centred offset (off = 8), and
    <= (2^(8-k) - 1/2 + 2^-14) s without it; the bounds are nearly reached (a wrong shift or
    offset breaks one side), and with off = 0 the reconstructions only grow with k (nesting)."""
    rng = np.random.default_rng(62)
    slack = 2.0 ** -14
    worst = {k: 0.0 for k in range(1, 8)}
    for x in random_groups(rng, 200, n):
        s, z, c = oracle.quantize_group(x)
        xf = x.astype(np.float64)
        prev = None
        for k in range(1, 9):
            rec = np.array([oracle.dequant_topk(ci, s, z, k, 8) for ci in c])
            e = np.max(np.abs(rec - xf)) / s
            bound = (2.0 ** (7 - k) if k < 8 else 0.0) + 0.5 + slack
            assert e <= bound, (k, e, bound)
            if k < 8:
                worst[k] = max(worst[k], e)
            rec0 = np.array([oracle.dequant_topk(ci, s, z, k, 0) for ci in c])
            assert np.max(np.abs(rec0 - xf)) / s <= 2.0 ** (8 - k) - 0.5 + slack
            if prev is not None:
                assert np.all(rec0 >= prev - 1e-12 * s)
            prev = rec0
    for k in range(1, 8):
        assert worst[k] >= 0.9 * 2.0 ** (7 - k), (k, worst[k])


@pytest.mark.parametrize("k,off,m16", [(2, 8, False), (2, 0, False), (3, 8, False), (2, 8, True),
                                       (1, 8, False)])
def test_topk_draft_equals_verify_when_the_low_bits_are_its_replacement(k, off, m16):
    """With the low 8 - k bits of every stored code set to the k-bit draft's replacement
    (off/16 of their range), every code is its own top-k reconstruction: a one-query verify then
    equals the k-bit draft exactly; before, the k-bit draft equals itself on the untouched cache
    (it reads only the top bits), and k = 4 / k = 8 equal the plain draft / verify."""
    H, D = 3, 64
    c = OracleCache(1, 2, H, D, G, 4 * G, 4, draft_offset=off, meta_fp16=m16)
    kk, vv = synth.kv_host(2, 2 * G + 50, H, D, 141, 142)
    c.prefill(0, kk, vv, n=[2 * G + 50, G + 7])
    q = synth.queries_host(2, None, H, D, 143, gain=2.0)
    assert np.array_equal(c.attend_draft_bits(0, q, 4), c.attend_draft(0, q))
    assert np.array_equal(c.attend_draft_bits(0, q, 8), c.attend_verify(0, q[:, None])[:, 0])
    before = c.attend_draft_bits(0, q, k)
    rep = (off << (8 - k)) >> 4
    c.set_low_bits(0, 8 - k, rep)
    draft = c.attend_draft_bits(0, q, k)
    assert np.array_equal(draft, before)
    assert np.array_equal(draft, c.attend_verify(0, q[:, None])[:, 0])
    c.set_low_bits(0, 8 - k, rep ^ 1)
    assert not np.array_equal(c.attend_verify(0, q[:, None])[:, 0], draft)


def test_topk_draft_over_explicit_dequantized_cache():
    """The 2-bit draft equals SDPA over keys / values dequantized here (with the pinned scalar
    dequant_topk) from the read-back codes and metadata, the fp16 tail appended."""
    B, H, D = 1, 2, 64
    c = OracleCache(1, B, H, D, G, 4 * G, 6)
    k, v = synth.kv_host(B, 3 * G + 21, H, D, 151, 152, outliers=synth.outlier_channels(H, D, 153))
    c.prefill(0, k, v)
    q = synth.queries_host(B, None, H, D, 154, gain=1.5)
    out = c.attend_draft_bits(0, q, 2, sm_scale=0.9)
    dq = np.vectorize(lambda c8, s, z: oracle.dequant_topk(int(c8), float(s), float(z), 2, 8))
    for h in range(H):
        ck = c.codes(0, 0, h)[:3 * G]
        cv = c.codes(0, 0, h, True)[:3 * G]
        km, vm = c.meta(0, 0, h)
        ks = np.repeat(km[:, :, 0], G, axis=0)[:3 * G]
        kz = np.repeat(km[:, :, 1], G, axis=0)[:3 * G]
        ka = np.concatenate([dq(ck, ks, kz), f64(k[0, 3 * G:, h])])
        va = np.concatenate([dq(cv, vm[:3 * G, 0:1], vm[:3 * G, 1:2]), f64(v[0, 3 * G:, h])])
        ref = sdpa(f64(q[0, h])[None], ka, va, scale=0.9)[0]
        assert np.max(np.abs(out[0, h] - ref)) < 1e-6


def test_upper_split_export_matches_the_codes():
    """The 2-bit planes of the split-upper layout hold C8 >> 6 (top) and (C8 >> 4) & 3
    (middle) of every code at the documented positions; 4 top + middle is the default layout's
    upper nibble."""
    B, H, D = 1, 2, 64
    c = OracleCache(1, B, H, D, G, 3 * G, 4)
    k, v = synth.kv_host(B, 2 * G + 9, H, D, 161, 162)
    c.prefill(0, k, v)
    sp = c.export_upper_split(0)
    img = c.export_layer(0)
    for h in range(H):
        ck = c.codes(0, 0, h).astype(np.int64)[:2 * G]
        cv = c.codes(0, 0, h, True).astype(np.int64)[:2 * G]
        # keys: token rows of D/4 bytes
        tw = sp["tk"][0, h, :2 * G].reshape(2 * G, D // 16, 4)
        mw = sp["mk"][0, h, :2 * G].reshape(2 * G, D // 16, 4)
        for wi in range(D // 16):
            w_t = tw[:, wi].astype(np.uint32) @ (1 << (8 * np.arange(4, dtype=np.uint32)))
            w_m = mw[:, wi].astype(np.uint32) @ (1 << (8 * np.arange(4, dtype=np.uint32)))
            for e in range(8):
                a, b = 16 * wi + e, 16 * wi + 8 + e
                assert np.array_equal((w_t >> (4 * e + 2)) & 3, ck[:, a] >> 6)
                assert np.array_equal((w_t >> (4 * e)) & 3, ck[:, b] >> 6)
                assert np.array_equal((w_m >> (4 * e)) & 3, (ck[:, a] >> 4) & 3)
                assert np.array_equal((w_m >> (4 * e + 2)) & 3, (ck[:, b] >> 4) & 3)
        # values: channel rows of G/8 bytes per half group
        for g in range(2):
            for e2 in range(2):
                tok = cv[g * G + e2 * G // 2: g * G + (e2 + 1) * G // 2]   # [G/2][D]
                for d in range(D):
                    tv = sp["tv"][0, h, g, e2, d].reshape(G // 32, 4).astype(np.uint32)
                    mv = sp["mv"][0, h, g, e2, d].reshape(G // 32, 4).astype(np.uint32)
                    wt = tv @ (1 << (8 * np.arange(4, dtype=np.uint32)))
                    wm = mv @ (1 << (8 * np.arange(4, dtype=np.uint32)))
                    for wi in range(G // 32):
                        for e in range(8):
                            a, b = 16 * wi + e, 16 * wi + 8 + e
                            assert (wt[wi] >> (4 * e + 2)) & 3 == tok[a, d] >> 6
                            assert (wt[wi] >> (4 * e)) & 3 == tok[b, d] >> 6
                            assert (wm[wi] >> (4 * e)) & 3 == (tok[a, d] >> 4) & 3
                            assert (wm[wi] >> (4 * e + 2)) & 3 == (tok[b, d] >> 4) & 3
        # 4 top + middle = the upper nibble of the default layout
        uk = img["uk"][0, h, :2 * G].astype(np.int64)
        assert np.array_equal(uk & 15, ck[:, 0::2] >> 4)
    # rows past nq are zero
    assert not sp["tk"][:, :, 2 * G:].any() and not sp["tv"][:, :, 2:].any()
