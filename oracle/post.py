"""Post-step updates (test infrastructure).

* SureLock lock rule (technical summary 2.1 item 1): a position locks once its
  local KL is at or below epsilon and, optionally, its confidence is high;
  locking is permanent (the locked set never shrinks).  Only positions whose
  statistics were recomputed this iteration are tested; a position without a
  previous posterior (first iteration) never locks.
* Confidence unmasking (ES-dLLM summary section 1; SureLock section 1): in
  each iteration the most confident masked positions of the current block are
  replaced by their argmax token; ties go to the lower index.
* Planned unmasking (DUS summary, technical summary section 2): the positions
  a dilated schedule assigns to the current round are unmasked together,
  whatever their confidence; the schedule marks them with force == 1.
"""
from __future__ import annotations

import numpy as np

from .selection import FORCE_EXCLUDED


def surelock_update(force: np.ndarray, rows: np.ndarray, conf: np.ndarray, kl: np.ndarray,
                    have_prev: bool, eps: float, conf_min: float) -> np.ndarray:
    """force: [N] uint8 (2 = locked); rows: flat positions recomputed this step."""
    out = np.array(force, copy=True)
    if not have_prev:
        return out
    for r in rows:
        if kl[r] <= eps and conf[r] > conf_min:
            out[r] = FORCE_EXCLUDED
    return out


def unmask_topn(tokens: np.ndarray, conf: np.ndarray, argmax: np.ndarray, mask_id: int,
                lo: int, hi: int, n: int) -> np.ndarray:
    """tokens/conf/argmax: [B, S].  Unmask the n most confident masked positions in [lo, hi)."""
    out = np.array(tokens, copy=True)
    B = tokens.shape[0]
    for b in range(B):
        cand = [i for i in range(lo, hi) if tokens[b, i] == mask_id]
        cand.sort(key=lambda i: (-float(conf[b, i]), i))
        for i in cand[:n]:
            out[b, i] = argmax[b, i]
    return out


def unmask_forced(tokens: np.ndarray, force: np.ndarray, argmax: np.ndarray, mask_id: int,
                  lo: int, hi: int) -> np.ndarray:
    """tokens/force/argmax: [B, S].  Unmask every masked position of [lo, hi) with force == 1."""
    out = np.array(tokens, copy=True)
    B = tokens.shape[0]
    for b in range(B):
        for i in range(lo, hi):
            if tokens[b, i] == mask_id and force[b, i] == 1:
                out[b, i] = argmax[b, i]
    return out
