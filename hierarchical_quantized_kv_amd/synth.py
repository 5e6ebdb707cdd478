"""Seeded synthetic inputs for the cache: fp16 keys, values, queries and acceptance draws.

These stand in for the key/value activations of Llama-2-7B-32K / LWM-Text-Chat-128k on long
documents, which are not available: only the shapes, the value distributions (N(0,1), 1 % of
key channels scaled by 8 as outliers, Student-t(3) keys for the stress case) and the speculation
pattern (Bernoulli(0.9) per drafted token, first rejection ends the round) are reproduced.

This module holds none of the cache's arithmetic.  Both the GPU library and the CPU oracle are
fed from it.  Two back ends give the same distributions:
  * numpy (PCG64), on the host, for test-sized inputs;
  * torch on a device (its Philox generator), for full-size inputs; callers copy the slices the
    oracle needs back to the host.
"""
from __future__ import annotations

import math

import numpy as np

OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 8.0


def seed_for(config: int, layer: int, stream: str) -> int:
    """Independent seed per (config, layer, stream); stream names the tensor ('k', 'v', 'q', ...)."""
    tag = {"k": 1, "v": 2, "q": 3, "accept": 4, "outlier": 5, "len": 6}[stream]
    return (1000 * config + layer) * 16 + tag


def outlier_channels(H: int, D: int, seed: int, frac: float = OUTLIER_FRACTION) -> np.ndarray:
    """round(frac * H * D) distinct (head, channel) pairs chosen by a seeded permutation."""
    n = int(round(frac * H * D))
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(H * D)[:n]
    return np.stack([perm // D, perm % D], axis=1).astype(np.int64)


def _student_t3(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape)
    chi2 = (rng.standard_normal((3,) + tuple(shape)) ** 2).sum(axis=0)
    return z / np.sqrt(chi2 / 3.0)


def kv_host(B: int, n: int, H: int, D: int, seed_k: int, seed_v: int, dist_k: str = "normal",
            outliers: np.ndarray | None = None):
    """Host fp16 keys and values [B][n][H][D]."""
    rk = np.random.Generator(np.random.PCG64(seed_k))
    rv = np.random.Generator(np.random.PCG64(seed_v))
    if dist_k == "student_t3":
        k = _student_t3(rk, (B, n, H, D))
    else:
        k = rk.standard_normal((B, n, H, D))
    if outliers is not None and len(outliers):
        k[:, :, outliers[:, 0], outliers[:, 1]] *= OUTLIER_GAIN
    v = rv.standard_normal((B, n, H, D))
    return k.astype(np.float16), v.astype(np.float16)


def queries_host(B: int, m: int | None, H: int, D: int, seed: int, gain: float = 1.0):
    """Host fp16 queries ~ N(0, 1) / sqrt(D) (times gain): [B][H][D], or [B][m][H][D]."""
    r = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, D) if m is None else (B, m, H, D)
    return (r.standard_normal(shape) * (gain / math.sqrt(D))).astype(np.float16)


def acceptance(rng: np.random.Generator, gamma: int, p: float = 0.9) -> int:
    """Number of accepted draft tokens: sequential Bernoulli(p) draws until the first rejection."""
    a = 0
    while a < gamma and rng.random() < p:
        a += 1
    return a


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-sequence lengths drawn uniformly from the integers lo .. hi inclusive."""
    return np.random.Generator(np.random.PCG64(seed)).integers(lo, hi + 1, size=B)


# ----------------------------------------------------------------------------------------------
# Device back end (torch), for inputs too large to generate on the host.
# ----------------------------------------------------------------------------------------------

def kv_device(torch, B: int, n: int, H: int, D: int, seed_k: int, seed_v: int, device,
              dist_k: str = "normal", outliers: np.ndarray | None = None):
    """Device fp16 keys and values [B][n][H][D] from torch's seeded device generator."""
    gk = torch.Generator(device=device).manual_seed(seed_k)
    gv = torch.Generator(device=device).manual_seed(seed_v)
    if dist_k == "student_t3":
        z = torch.randn((B, n, H, D), generator=gk, device=device, dtype=torch.float32)
        chi2 = torch.zeros_like(z)
        for _ in range(3):
            chi2 += torch.randn((B, n, H, D), generator=gk, device=device,
                                dtype=torch.float32) ** 2
        k = z / torch.sqrt(chi2 / 3.0)
        del z, chi2
    else:
        k = torch.randn((B, n, H, D), generator=gk, device=device, dtype=torch.float32)
    if outliers is not None and len(outliers):
        hh = torch.as_tensor(outliers[:, 0], device=device)
        dd = torch.as_tensor(outliers[:, 1], device=device)
        k[:, :, hh, dd] *= OUTLIER_GAIN
    k = k.to(torch.float16)
    v = torch.randn((B, n, H, D), generator=gv, device=device, dtype=torch.float32).to(
        torch.float16)
    return k, v
