"""Shared helpers of the GPU parity tests."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

DEV = "cuda"

# Element-wise relative errors are taken against max(|o_i|, ELEM_FLOOR * max|o|).
ELEM_FLOOR = 1e-3
# When this variable names a file, every assert_close appends one JSON line to it (the
# element-wise report); pytest's output capture would otherwise hide the printed line.
REPORT_ENV = "DLLM_PARITY_REPORT"


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def max_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max_i |g_i - o_i| / max_i |o_i| (infinity-norm relative error)."""
    den = float(np.max(np.abs(want)))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / den)


def elem_rel_err(got: np.ndarray, want: np.ndarray, floor: float = ELEM_FLOOR) -> np.ndarray:
    """|g_i - o_i| / max(|o_i|, floor * max|o|) for every element (0 where both are 0)."""
    a = np.abs(want)
    den = np.maximum(a, floor * float(np.max(a)) if a.size else 0.0)
    diff = np.abs(got - want)
    out = np.zeros_like(diff)
    nz = den > 0
    out[nz] = diff[nz] / den[nz]
    out[~nz] = diff[~nz]
    return out


def elem_report(got: np.ndarray, want: np.ndarray, what: str, tol: float) -> dict:
    """The element-wise report: worst and 99.9th-percentile floored relative error, the share of
    elements above the infinity-norm tolerance, and where the worst element sits."""
    e = elem_rel_err(got, want)
    flat = e.reshape(-1)
    worst = int(np.argmax(flat)) if flat.size else 0
    rep = {"what": what, "n": int(flat.size), "inf_norm": max_rel_err(got, want),
           "elem_max": float(flat[worst]) if flat.size else 0.0,
           "elem_p999": float(np.quantile(flat, 0.999)) if flat.size else 0.0,
           "elem_frac_over_tol": float(np.mean(flat > tol)) if flat.size else 0.0,
           "worst_index": worst,
           "worst_want": float(want.reshape(-1)[worst]) if flat.size else 0.0,
           "max_abs_want": float(np.max(np.abs(want))) if flat.size else 0.0}
    path = os.environ.get(REPORT_ENV)
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], **rep}) + "\n")
    return rep


def assert_close(got, want, tol: float, what: str, etol: float | None = None):
    """Asserts the infinity-norm relative error <= tol and, with `etol`, every element's floored
    relative error <= etol; the element-wise report is printed (and logged under REPORT_ENV)."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    rep = elem_report(g, w, what, tol)
    print(f"{what}: inf-norm {rep['inf_norm']:.3e}, element-wise max {rep['elem_max']:.3e} "
          f"(p99.9 {rep['elem_p999']:.3e}, {100 * rep['elem_frac_over_tol']:.3f}% over {tol:.0e})")
    assert rep["inf_norm"] <= tol, f"{what}: max relative error {rep['inf_norm']:.3e} > {tol:.1e}"
    if etol is not None:
        assert rep["elem_max"] <= etol, (f"{what}: element-wise relative error {rep['elem_max']:.3e} > {etol:.1e} "
                                         f"at flat index {rep['worst_index']} (want {rep['worst_want']:.4e})")
    return rep["inf_norm"]


def assert_within(got, want, bound, what: str):
    """Element-wise |g_i - o_i| <= bound_i (a bound derived for the quantity under test)."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    b = np.broadcast_to(np.asarray(bound, dtype=np.float64), w.shape)
    r = np.abs(g - w) / np.maximum(b, np.finfo(np.float64).tiny)
    worst = int(np.argmax(r))
    print(f"{what}: worst |g - o| / bound = {float(r.reshape(-1)[worst]):.3f}")
    assert np.all(np.abs(g - w) <= b), (f"{what}: |g - o| = {abs(g.reshape(-1)[worst] - w.reshape(-1)[worst]):.3e} "
                                        f"> bound {b.reshape(-1)[worst]:.3e} at flat index {worst}")


def kl_first_order(zc_g, zc_o, zp_g, zp_o, exclude):
    """The KL difference that the logit differences alone explain, and a bound on the rest.

    With D = z - z', p = softmax(z), p' = softmax(z'), the KL(p || p') changes to first order in the
    logit differences dz (current logits, GPU - oracle) and dz' (previous logits) by
        sum_v p_v (D_v - mean_p D) dz_v + sum_v (p'_v - p_v) dz'_v .
    Its second derivatives are bounded by (1 + 2 max|D - mean_p D|) for dz dz, 2 for dz dz' and
    1 for dz' dz' (each times a probability weight summing to 1), so the remainder is at most
    (1 + 2 max|D - mean_p D|) max|dz|^2 + 2 max|dz| max|dz'| + max|dz'|^2; the kernel's fp32
    arithmetic adds 1e-3 relative and 1e-6 absolute (as for the fp32 model).  Returns
    (first-order change, bound on |KL_gpu - KL_oracle - first-order change| without the relative part)."""
    keep = np.ones(zc_o.shape[1], dtype=bool)
    if exclude >= 0:
        keep[exclude] = False
    zc, zp = zc_o[:, keep], zp_o[:, keep]
    p = np.exp(zc - zc.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pp = np.exp(zp - zp.max(axis=1, keepdims=True))
    pp /= pp.sum(axis=1, keepdims=True)
    dlt = zc - zp
    dev = dlt - np.sum(p * dlt, axis=1, keepdims=True)
    dz = zc_g[:, keep] - zc
    dzp = zp_g[:, keep] - zp
    first = np.sum(p * dev * dz, axis=1) + np.sum((pp - p) * dzp, axis=1)
    a, b = np.max(np.abs(dz), axis=1), np.max(np.abs(dzp), axis=1)
    second = (1 + 2 * np.max(np.abs(dev), axis=1)) * a * a + 2 * a * b + b * b
    return first, second + 1e-6


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
