"""Rounding helpers of the oracle (test infrastructure).

bf16 storage: the GPU keeps activations, caches and weights as bf16 with fp32
arithmetic in between.  The oracle mirrors the *storage* points only: a
float64 value is rounded once, round-to-nearest-even, to the bf16 grid.
"""
from __future__ import annotations

import numpy as np

_BF16_MANT = 7          # explicit mantissa bits of bf16
_BF16_EMIN = -126       # smallest normal exponent (shared with fp32)
_BF16_MAX_EXP = 128     # values >= 2**128 after rounding overflow to inf


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    Exact: the value is divided by its bf16 spacing (a power of two, so the
    division is exact), rounded half-to-even by ``np.rint``, and scaled back.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, ex = np.frexp(xf)                     # xf = m * 2**ex, 0.5 <= |m| < 1
    e = np.maximum(ex - 1, _BF16_EMIN)       # binade exponent, clamped to subnormal range
    spacing_exp = e - _BF16_MANT
    r = np.ldexp(np.rint(np.ldexp(xf, -spacing_exp)), spacing_exp)
    r = np.where(np.abs(r) >= 2.0 ** _BF16_MAX_EXP, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def fl32(x) -> np.ndarray:
    """Round float64 values to fp32 (RNE) and return them as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store_fn(mode: str):
    """Rounding applied at a storage point: bf16 in "bf16" mode, none in "exact"."""
    if mode == "bf16":
        return round_bf16
    if mode == "exact":
        return lambda v: np.asarray(v, dtype=np.float64)
    raise ValueError(f"unknown precision mode {mode!r}")
