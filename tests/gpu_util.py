"""Shared helpers of the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max_i |g_i - o_i| / max_i |o_i| (infinity-norm relative error)."""
    den = float(np.max(np.abs(want)))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / den)


def assert_close(got, want, tol: float, what: str):
    err = max_rel_err(np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64))
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol:.1e}"
    return err


def selection_gap(scores: np.ndarray, force: np.ndarray | None, k: int) -> float:
    """Score gap at the k boundary among free candidates (inf if the boundary is not between free rows)."""
    s = np.asarray(scores, dtype=np.float64)
    f = np.zeros(len(s), dtype=np.uint8) if force is None else np.asarray(force)
    n_forced = int(np.sum(f == 1))
    free = np.sort(s[(f == 0) & ~np.isnan(s)])[::-1]
    kk = k - n_forced
    if kk <= 0 or kk >= len(free):
        return float("inf")
    return float(free[kk - 1] - free[kk])
