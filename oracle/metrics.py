"""Comparison metrics for the parity tests (test infrastructure only).

The numerical report fields follow the review's reproduction notes (cosine,
relative L2, max-abs, per-row error, code underflow) and its small-gradient
example in "Small gradients deserve a metric of their own" (one entry 1 and
100 entries 0.001: dropping the small ones costs about 1 % relative L2 error
and leaves cosine near 0.99995, so a zero-fraction count is reported too).
"""
from __future__ import annotations

import numpy as np


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def max_abs(got, ref) -> float:
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(d.max()) if d.size else 0.0


def row_rel_err(got, ref, floor_frac: float = 1e-3) -> np.ndarray:
    """Per-row max relative error over the last axis:
    max_c |got - ref| / max(max_c |ref|, floor_frac * max |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return np.zeros(0)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    floor = floor_frac * float(np.abs(r).max()) if r.size else 0.0
    denom = np.maximum(np.abs(r).max(axis=1), floor)
    num = np.abs(g - r).max(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(denom > 0, num / np.where(denom > 0, denom, 1.0), num)
    return out


def zero_fraction(got, ref) -> float:
    """Fraction of entries nonzero in ref that are zero in got."""
    got = np.asarray(got).ravel()
    ref = np.asarray(ref).ravel()
    nz = ref != 0
    return float(np.mean(got[nz] == 0)) if nz.any() else 0.0


def report(got, ref) -> dict:
    rr = row_rel_err(got, ref)
    return {
        "cos": cosine(got, ref),
        "rel_l2": rel_l2(got, ref),
        "max_abs": max_abs(got, ref),
        "max_ref": float(np.abs(np.asarray(ref, dtype=np.float64)).max()) if np.size(ref) else 0.0,
        "row_rel_max": float(rr.max()) if rr.size else 0.0,
        "zero_frac": zero_fraction(got, ref),
    }
