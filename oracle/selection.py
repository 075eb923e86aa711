"""Active-row selection (test infrastructure).

ES-dLLM (technical summary 2.1 item 2) keeps the top-k positions by
importance and skips the rest; dLLM-Cache (explainer section 3) recomputes a
response row only when its similarity to the cached value is low, with an
update ratio rho (section 4); SureLock (technical summary 2.1 item 2) removes
locked positions from all later computation.

Total order used (the pages fix none; ties go to the lower index):
  1. forced rows (force == 1) first,
  2. then non-NaN scores before NaN scores,
  3. then higher score first (-0.0 and +0.0 compare equal),
  4. then lower index first.
Rows with force == 2 (locked / excluded) are never candidates.  The selected
set is the first k rows of this order; it is returned in ascending index order.
This module defines the order by counting, for each row, how many candidates
precede it: a row is selected iff fewer than k rows precede it.
"""
from __future__ import annotations

import numpy as np

FORCE_NONE, FORCE_ON, FORCE_EXCLUDED = 0, 1, 2


def order_before(si: float, fi: bool, i: int, sj: float, fj: bool, j: int) -> bool:
    """True iff row i precedes row j in the selection order."""
    if fi != fj:
        return fi
    if fi:
        return i < j
    ni, nj = np.isnan(si), np.isnan(sj)
    if ni != nj:
        return nj
    if not ni and si != sj:
        return si > sj
    return i < j


def _ranks(scores: np.ndarray, force: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Number of candidates preceding each candidate (vectorised counting)."""
    s = np.asarray(scores, dtype=np.float64)
    f = np.asarray(force)
    cand = f != FORCE_EXCLUDED
    forced = (f == FORCE_ON) & cand
    nan = np.isnan(s)
    sv = np.where(nan, 0.0, s) + 0.0          # -0.0 -> +0.0
    n = s.size
    idx = np.arange(n)
    # before[j, i]: candidate j precedes candidate i
    fj, fi = forced[:, None], forced[None, :]
    nj, ni = nan[:, None], nan[None, :]
    sj, si = sv[:, None], sv[None, :]
    jj, ii = idx[:, None], idx[None, :]
    both_forced = fj & fi
    both_free = ~fj & ~fi
    free_order = (~nj & ni) | ((nj == ni) & ((~nj & (sj > si)) | ((nj | (sj == si)) & (jj < ii))))
    before = (fj & ~fi) | (both_forced & (jj < ii)) | (both_free & free_order)
    before &= cand[:, None] & cand[None, :]
    return before.sum(axis=0), cand


def select_topk(scores: np.ndarray, force: np.ndarray | None, k: int) -> np.ndarray:
    """Ascending indices of the first k candidates of the selection order."""
    n = len(scores)
    if force is None:
        force = np.zeros(n, dtype=np.uint8)
    rank, cand = _ranks(scores, force)
    sel = cand & (rank < k)
    return np.nonzero(sel)[0].astype(np.int64)


def select_thresh_cap(scores: np.ndarray, force: np.ndarray | None, tau: float, k: int) -> np.ndarray:
    """Rows that are forced or score strictly above tau, capped at k by the order."""
    n = len(scores)
    if force is None:
        force = np.zeros(n, dtype=np.uint8)
    s = np.asarray(scores, dtype=np.float64)
    f = np.asarray(force)
    qualifies = (f != FORCE_EXCLUDED) & ((f == FORCE_ON) | (s > tau))
    k_eff = min(int(k), int(qualifies.sum()))
    return select_topk(scores, force, k_eff)
