"""Tolerance of the attention outputs against the CPU oracle (numpy only, no GPU).

Two bounds, both asserted:
  * max |got - ref| <= ATOL = 2e-3 over the whole output (fp32 accumulation over dequantized
    values);
  * per output row (one (sequence, query, head): its D channels), max |got - ref| / max |ref|
    <= RTOL_ROW = 1e-3.  The split-softmax merge is exact in real arithmetic, so only rounding
    separates the two results; at long contexts |out| is a few 1e-3, where the absolute bound
    alone would let a dropped or doubled group through (tests/test_parity_gate.py shows the
    row bound catching both).
"""
from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL_ROW = 1e-3


def compare(got, ref):
    """(max abs error, worst per-row relative error) of got against ref (same shape, last axis
    the channels)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != {ref.shape}")
    d = np.abs(got - ref)
    if d.size == 0:
        return 0.0, 0.0
    mad = float(d.max())
    rows_d = d.reshape(-1, d.shape[-1]).max(axis=1)
    rows_r = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    rel = float(np.max(rows_d / np.maximum(rows_r, 1e-30)))
    return mad, rel


def check_close(got, ref, what=""):
    """Asserts both bounds; returns (max abs error, worst row relative error)."""
    g = np.asarray(got)
    if not np.all(np.isfinite(g)):
        raise AssertionError(f"{what}: non-finite output")
    mad, rel = compare(g, ref)
    if mad > ATOL:
        raise AssertionError(f"{what}: max abs err {mad:.3e} > {ATOL} (row rel {rel:.3e})")
    if rel > RTOL_ROW:
        raise AssertionError(f"{what}: row relative err {rel:.3e} > {RTOL_ROW} (abs {mad:.3e})")
    return mad, rel
