"""Per-position posterior statistics from the LM-head logits (test infrastructure).

* confidence: the largest softmax probability of the row (ES-dLLM summary:
  tokens are unmasked in order of confidence, and Eq. 1 reuses the previous
  iteration's confidence c_i^(t-1));
* argmax: the token that unmasking would write (lowest id on ties);
* local KL: D_t^(i) = KL(p_t^(i) || p_{t-1}^(i)), natural log, between this
  iteration's and the previous iteration's posterior of the same position
  (SureLock technical summary 2.1 item 1).

The mask token's logit is excluded (treated as -inf) when ``exclude_id >= 0``,
so a position is never "unmasked" to the mask token.  KL uses the form
sum_v p_v * ((z_v - z'_v) - (lse - lse')), clamped at 0, which is exactly 0
for identical logits.
"""
from __future__ import annotations

import numpy as np


def _lse(z: np.ndarray) -> tuple[float, float]:
    m = float(np.max(z))
    return m, m + float(np.log(np.sum(np.exp(z - m))))


def conf_kl_row(z: np.ndarray, z_prev: np.ndarray | None, exclude_id: int = -1):
    """(conf, argmax, kl) of one row of logits; kl is +inf without previous logits."""
    z = np.asarray(z, dtype=np.float64)
    keep = np.ones(z.size, dtype=bool)
    if exclude_id >= 0:
        keep[exclude_id] = False
    zk = z[keep]
    ids = np.nonzero(keep)[0]
    m, lse = _lse(zk)
    conf = float(np.exp(m - lse))
    argmax = int(ids[np.nonzero(zk == m)[0][0]])
    if z_prev is None:
        return conf, argmax, float("inf")
    zp = np.asarray(z_prev, dtype=np.float64)[keep]
    _, lse_p = _lse(zp)
    p = np.exp(zk - lse)
    kl = float(np.sum(p * ((zk - zp) - (lse - lse_p))))
    return conf, argmax, max(0.0, kl)


def conf_kl(logits: np.ndarray, logits_prev: np.ndarray | None, exclude_id: int = -1):
    """Row-wise conf [R], argmax [R], kl [R] (kl = +inf when logits_prev is None)."""
    R = logits.shape[0]
    conf = np.empty(R)
    arg = np.empty(R, dtype=np.int64)
    kl = np.empty(R)
    for r in range(R):
        conf[r], arg[r], kl[r] = conf_kl_row(logits[r], None if logits_prev is None else logits_prev[r], exclude_id)
    return conf, arg, kl
