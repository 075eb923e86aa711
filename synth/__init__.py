"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and bench.py.

This module holds no arithmetic of the denoising method: it only draws numbers.
Every value is a pure function of (seed tuple, element index), computed with a
32-bit integer hash and exact integer sums, so the same call yields the same
bits on the host (torch CPU) and on the device (torch CUDA/HIP).

Distributions
-------------
* ``normal``: a scaled Irwin-Hall sum of four independent 16-bit uniforms
  (mean 0, the requested standard deviation, support +-3.46 sigma).  The
  integer sum is exact, its conversion to fp32 is exact (|z| < 2**24), and the
  single fp32 multiply by the scale is correctly rounded on every IEEE device,
  so host and device agree bit for bit, also after RNE rounding to bf16.
* ``uniform01``: 24-bit uniforms ``k * 2**-24`` on [0, 1).
* ``randint``: ``hash % n`` (the modulo bias is below 2**-15 for the vocabulary
  sizes used here).

The hash is "lowbias32" (two multiply-xorshift rounds, public domain).
"""
from __future__ import annotations

import torch

__all__ = ["seed_of", "normal", "uniform01", "randint", "hash32"]

_MASK32 = 0xFFFFFFFF
# Irwin-Hall(4) over {0..65535}: variance = 4 * (65536**2 - 1) / 12
_IH4_STD = (4.0 * (65536.0 ** 2 - 1.0) / 12.0) ** 0.5
_IH4_MEAN = 2 * 65535
_CHUNK = 1 << 26


def hash32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 on int64 tensors holding values in [0, 2**32)."""
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & _MASK32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & _MASK32
    x = x ^ (x >> 16)
    return x


def seed_of(*parts: int) -> int:
    """Fold a tuple of small non-negative ints into one 32-bit seed."""
    s = 0x9E3779B9
    for p in parts:
        t = torch.tensor([(s ^ (int(p) & _MASK32)) & _MASK32], dtype=torch.int64)
        s = int(hash32(t + 0x632BE5AB)[0]) ^ ((s << 6) & _MASK32) ^ (s >> 2)
        s &= _MASK32
    return s


def _words(seed: int, start: int, count: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    sh = int(hash32(torch.tensor([seed], dtype=torch.int64))[0])
    h1 = hash32(((2 * i) & _MASK32) ^ sh)
    h2 = hash32(((2 * i + 1) & _MASK32) ^ sh)
    return h1, h2


def normal(seed: int, shape, std: float, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0, std) stand-in (scaled Irwin-Hall of four 16-bit uniforms)."""
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=dtype, device=device)
    scale = torch.tensor(float(std) / _IH4_STD, dtype=torch.float32).item()
    for start in range(0, n, _CHUNK):
        c = min(_CHUNK, n - start)
        h1, h2 = _words(seed, start, c, device)
        z = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16) - _IH4_MEAN
        del h1, h2
        v = z.to(torch.float32) * torch.tensor(scale, dtype=torch.float32, device=device)
        out[start:start + c] = v.to(dtype)
    return out.view(*[int(s) for s in shape])


def uniform01(seed: int, shape, device="cpu") -> torch.Tensor:
    """fp32 uniforms k * 2**-24, k in [0, 2**24)."""
    n = 1
    for s in shape:
        n *= int(s)
    h1, _ = _words(seed, 0, n, device)
    return ((h1 >> 8).to(torch.float32) * (2.0 ** -24)).view(*[int(s) for s in shape])


def randint(seed: int, shape, n_values: int, device="cpu") -> torch.Tensor:
    """int32 values in [0, n_values)."""
    n = 1
    for s in shape:
        n *= int(s)
    h1, _ = _words(seed, 0, n, device)
    return (h1 % int(n_values)).to(torch.int32).view(*[int(s) for s in shape])


def permutation(seed: int, n: int, device="cpu") -> torch.Tensor:
    """A seeded permutation of range(n): argsort of distinct 64-bit hash keys."""
    h1, h2 = _words(seed, 0, n, device)
    key = (h1 << 31) ^ h2  # < 2**63, ties broken by stable sort on index
    return torch.sort(key, stable=True).indices.to(torch.int64)
