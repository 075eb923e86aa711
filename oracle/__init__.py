"""CPU oracle for one token-skipping denoising iteration (TEST INFRASTRUCTURE).

This package is the plain, slow, obviously-correct reference against which the
HIP library is checked.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does, and it imports nothing from the product package.

It is written in NumPy, in float64, from the descriptions on these pages:

* ES-dLLM, "Efficient Inference for Diffusion Large Language Models by
  Early-Skipping" (gist.science summary, technical summary section 2.1:
  importance score Eq. 1; partial cache update and early skip).
* SureLock, "Stopping Computation for Converged Tokens in Masked Diffusion-LM
  Decoding" (gist.science summary, technical summary section 2.1: local KL
  lock rule; locked rows stay attendable through cached K/V).
* dLLM-Cache (aibr.jp explainer, section 3: similarity-gated partial response
  update; section 4: update ratio).
* DUS, "Plan for Speed: Dilated Scheduling for Masked Diffusion Language
  Models" (gist.science summary, technical summary section 2: dilated
  coarse-to-fine rounds, R = ceil(log_a B)).

Precision modes: ``"exact"`` keeps every intermediate in float64;
``"bf16"`` rounds to bf16 (round-to-nearest-even, done on the float64 value)
at the storage points the GPU uses -- residual stream, normalised GEMM inputs,
Q/K/V and the caches, attention output, SiLU*mul output -- and to fp32 where
the GPU stores fp32 (logits, scores, statistics).  Everything between two
storage points is float64.

Parity status: every function is pinned by the ``-m "not gpu"`` tests under
``tests/`` (closed forms, invariants, brute force and library routines); none
is "parity unpinned".
"""
from .numerics import round_bf16, fl32, store_fn  # noqa: F401
from .transformer import (  # noqa: F401
    rmsnorm, rope, attention_rows, silu, layer_rows, dense_forward, lm_logits,
)
from .importance import psi, importance_score  # noqa: F401
from .selection import order_before, select_topk, select_thresh_cap  # noqa: F401
from .vocab import conf_kl_row, conf_kl  # noqa: F401
from .post import surelock_update, unmask_forced, unmask_topn  # noqa: F401
from .dus import dus_rounds  # noqa: F401
from .step import OracleModel, OracleState, StepCfg, ScoreCfg, skip_step, new_state  # noqa: F401
