"""Shapes and seeded random-init tensors of the five synthetic workloads.

No denoising arithmetic lives here: only dimensions and draws from ``synth``.
Weights follow nn.Linear layout ``[out_features, in_features]``, drawn
N(0, 0.02) (Irwin-Hall stand-in), norm gains are ones, and the mask token is
the last vocabulary id.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import normal, randint, seed_of


@dataclass(frozen=True)
class Dims:
    name: str
    cfg_id: int
    n_layers: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    B: int
    S: int
    prompt: int
    dtype: str  # "f32" or "bf16"

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


TINY = Dims("tiny_fp32_2L_d256", 1, 2, 256, 4, 4, 64, 768, 1024, 1, 128, 64, "f32")
LLADA_LAYER = Dims("llada8b_one_layer_s512", 2, 1, 4096, 32, 32, 128, 12288, 126464, 1, 512, 256, "bf16")
LLADA = Dims("llada8b_32L_s512_b1", 3, 32, 4096, 32, 32, 128, 12288, 126464, 1, 512, 256, "bf16")
DREAM = Dims("dream7b_28L_s1024_b8", 4, 28, 3584, 28, 4, 128, 18944, 152064, 8, 1024, 512, "bf16")
LLADA_LONG = Dims("llada8b_32L_s4096_b4", 5, 32, 4096, 32, 32, 128, 12288, 126464, 4, 4096, 3584, "bf16")

ALL = (TINY, LLADA_LAYER, LLADA, DREAM, LLADA_LONG)

# tensor ids inside one layer's seed tuple
T_EMBED, T_Q, T_K, T_V, T_O, T_GATE, T_UP, T_DOWN, T_LM = range(9)
WEIGHT_STD = 0.02


def shrink(base: Dims, **kw) -> Dims:
    """Same workload family with some dimensions replaced (for small tests)."""
    fields = dict(base.__dict__)
    fields.update(kw)
    return Dims(**fields)


def torch_dtype(dims: Dims):
    return torch.float32 if dims.dtype == "f32" else torch.bfloat16


def layer_weights(dims: Dims, layer: int, device="cpu", seed_base: int | None = None,
                  std: float = WEIGHT_STD) -> dict:
    """Separate per-layer tensors, each in the storage dtype of the workload."""
    cid = dims.cfg_id if seed_base is None else seed_base
    dt = torch_dtype(dims)
    Hq, Hkv, D, d, F = dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.d, dims.d_ff

    def w(tid, shape):
        return normal(seed_of(cid, layer, tid), shape, std, dt, device)

    return {
        "attn_norm": torch.ones(d, dtype=dt, device=device),
        "wq": w(T_Q, (Hq * D, d)),
        "wk": w(T_K, (Hkv * D, d)),
        "wv": w(T_V, (Hkv * D, d)),
        "wo": w(T_O, (d, Hq * D)),
        "ffn_norm": torch.ones(d, dtype=dt, device=device),
        "wg": w(T_GATE, (F, d)),
        "wu": w(T_UP, (F, d)),
        "wd": w(T_DOWN, (d, F)),
    }


def model_weights(dims: Dims, device="cpu", seed_base: int | None = None, std: float = WEIGHT_STD) -> dict:
    cid = dims.cfg_id if seed_base is None else seed_base
    dt = torch_dtype(dims)
    return {
        "embed": normal(seed_of(cid, 10_000, T_EMBED), (dims.vocab, dims.d), std, dt, device),
        "layers": [layer_weights(dims, l, device, seed_base, std) for l in range(dims.n_layers)],
        "final_norm": torch.ones(dims.d, dtype=dt, device=device),
        "lm_head": normal(seed_of(cid, 10_000, T_LM), (dims.vocab, dims.d), std, dt, device),
    }


def initial_tokens(dims: Dims, device="cpu", seed_base: int | None = None) -> torch.Tensor:
    """Prompt tokens uniform in [0, V-1) followed by mask tokens, [B, S] int32."""
    cid = dims.cfg_id if seed_base is None else seed_base
    tok = randint(seed_of(cid, 20_000), (dims.B, dims.S), dims.vocab - 1, device)
    tok[:, dims.prompt:] = dims.mask_id
    return tok.contiguous()
