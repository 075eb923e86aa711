"""Importance score of every position (test infrastructure).

ES-dLLM (gist.science summary, technical summary 2.1 item 1, Eq. 1): the
importance of position i is a weighted sum of the previous iteration's
confidence c_i^(t-1) and the relative change of an intermediate tensor,

    I_i = alpha * c_i + (1 - alpha) * ||H_i^(t) - H_i^(t-1)||_1 / (sqrt(d) * ||H_i^(t-1)||_2).

The change term may also be the cosine change of dLLM-Cache (aibr.jp
explainer, section 3: similarity-gated reuse), the relative L2 change, or the
previous step's local KL of SureLock (technical summary 2.1 item 1).  The
confidence enters either as c (Eq. 1 as printed) or as 1 - c
(``conf_inverted``), which is how the tiny workload states it.

Readings where the pages are silent:
* 1 - cos is evaluated as 0.5 * || a/|a| - b/|b| ||^2, which is exactly 0 for
  identical inputs.
* A zero-norm previous row (or a zero-norm current row for the cosine) gives
  psi = 0 if the two rows are identical and FLT_MAX otherwise.
* The final score is rounded to fp32, the precision the selection runs in.
"""
from __future__ import annotations

import numpy as np

from .numerics import fl32

VAR_L1N, VAR_COS, VAR_L2REL, VAR_KL, VAR_NONE = 0, 1, 2, 3, 4
FLT_MAX = float(np.finfo(np.float32).max)


def psi(h_cur: np.ndarray, h_prev: np.ndarray, var: int, kl_prev: float = 0.0) -> float:
    """Change term of one row (float64 inputs holding the stored values)."""
    if var == VAR_NONE:
        return 0.0
    if var == VAR_KL:
        return float(kl_prev)
    a = np.asarray(h_cur, dtype=np.float64)
    b = np.asarray(h_prev, dtype=np.float64)
    same = bool(np.array_equal(a, b))
    nb = float(np.sqrt(np.sum(b * b)))
    if var == VAR_L1N:
        if nb == 0.0:
            return 0.0 if same else FLT_MAX
        return float(np.sum(np.abs(a - b)) / (np.sqrt(a.size) * nb))
    if var == VAR_L2REL:
        if nb == 0.0:
            return 0.0 if same else FLT_MAX
        return float(np.sqrt(np.sum((a - b) ** 2)) / nb)
    if var == VAR_COS:
        na = float(np.sqrt(np.sum(a * a)))
        if na == 0.0 or nb == 0.0:
            return 0.0 if same else FLT_MAX
        diff = a / na - b / nb
        return float(0.5 * np.sum(diff * diff))
    raise ValueError(f"unknown variation kind {var}")


def importance_score(h_cur: np.ndarray, h_prev: np.ndarray, conf_prev: np.ndarray,
                     kl_prev: np.ndarray | None, *, alpha: float, var: int,
                     conf_inverted: bool) -> np.ndarray:
    """fp32 scores of all rows.  h_cur/h_prev: [N, w]; conf_prev/kl_prev: [N]."""
    N = h_cur.shape[0]
    out = np.empty(N, dtype=np.float64)
    for i in range(N):
        c = float(conf_prev[i])
        phi = 1.0 - c if conf_inverted else c
        p = psi(h_cur[i], h_prev[i], var, 0.0 if kl_prev is None else kl_prev[i])
        out[i] = alpha * phi + (1.0 - alpha) * p
    return fl32(out)
