"""Test helpers: converting seeded synthetic tensors into oracle inputs."""
from __future__ import annotations

import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_weights(w: dict) -> dict:
    """synth.workloads.model_weights(...) -> float64 NumPy dict for the oracle."""
    return {
        "embed": to_np(w["embed"]),
        "layers": [{k: to_np(v) for k, v in lw.items()} for lw in w["layers"]],
        "final_norm": to_np(w["final_norm"]),
        "lm_head": to_np(w["lm_head"]),
    }
