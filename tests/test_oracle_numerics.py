"""Pins for the oracle's rounding helpers (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.numerics import fl32, round_bf16


def test_round_bf16_matches_torch_on_fp32_values():
    # torch's fp32 -> bf16 conversion is round-to-nearest-even: a library routine.
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_ties_to_even_and_specials():
    one = 1.0
    assert round_bf16(one + 2.0 ** -8) == 1.0                      # halfway, even is 1.0
    assert round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6      # halfway, even is 1+2^-6
    assert round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert round_bf16(-(one + 2.0 ** -8)) == -1.0
    assert np.isinf(round_bf16(3.5e38))
    assert np.isnan(round_bf16(np.nan))
    assert round_bf16(0.0) == 0.0 and np.signbit(round_bf16(-0.0))


def test_fl32_is_fp32_rounding():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    np.testing.assert_array_equal(fl32(x), x.astype(np.float32).astype(np.float64))
    assert fl32(1.0 + 2.0 ** -24)[()] == 1.0
