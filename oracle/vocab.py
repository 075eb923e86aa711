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

Compact KL state (a reading; the pages fix no precision for it): the previous
logits may be kept rounded to bf16.  The KL then compares the bf16-rounded
current logits with the stored ones, KL(softmax(bf16(z)) || softmax(z')), so
identical logits still give exactly 0; confidence and argmax always come from
the unrounded logits.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_bf16


def _lse(z: np.ndarray) -> tuple[float, float]:
    m = float(np.max(z))
    return m, m + float(np.log(np.sum(np.exp(z - m))))


def conf_kl_row(z: np.ndarray, z_prev: np.ndarray | None, exclude_id: int = -1, prev_bf16: bool = False):
    """(conf, argmax, kl) of one row of logits; kl is +inf without previous logits.

    With ``prev_bf16`` the previous logits are the bf16-stored state and the KL is taken between
    the bf16-rounded current logits and them."""
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
    zc, lse_c = zk, lse
    if prev_bf16:
        zc = round_bf16(zk)
        _, lse_c = _lse(zc)
    p = np.exp(zc - lse_c)
    kl = float(np.sum(p * ((zc - zp) - (lse_c - lse_p))))
    return conf, argmax, max(0.0, kl)


def conf_kl(logits: np.ndarray, logits_prev: np.ndarray | None, exclude_id: int = -1, prev_bf16: bool = False):
    """Row-wise conf [R], argmax [R], kl [R] (kl = +inf when logits_prev is None)."""
    R = logits.shape[0]
    conf = np.empty(R)
    arg = np.empty(R, dtype=np.int64)
    kl = np.empty(R)
    for r in range(R):
        conf[r], arg[r], kl[r] = conf_kl_row(logits[r], None if logits_prev is None else logits_prev[r], exclude_id,
                                             prev_bf16)
    return conf, arg, kl


def kl_state_value(logits: np.ndarray, prev_bf16: bool = False) -> np.ndarray:
    """What the KL state holds for these logits after the pass: the logits, or their bf16 rounding."""
    z = np.asarray(logits, dtype=np.float64)
    return round_bf16(z) if prev_bf16 else z.copy()
