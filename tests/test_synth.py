"""The seeded generators are deterministic and have the stated moments (CPU only)."""
import numpy as np
import torch

import synth
from synth import workloads


def test_normal_is_deterministic_and_chunk_independent():
    a = synth.normal(synth.seed_of(1, 2, 3), (1000,), 0.02)
    b = synth.normal(synth.seed_of(1, 2, 3), (1000,), 0.02)
    assert torch.equal(a, b)
    c = synth.normal(synth.seed_of(1, 2, 4), (1000,), 0.02)
    assert not torch.equal(a, c)


def test_normal_moments():
    x = synth.normal(synth.seed_of(7), (400000,), 0.02).double()
    assert abs(float(x.mean())) < 2e-4
    assert abs(float(x.std()) / 0.02 - 1.0) < 5e-3
    assert float(x.abs().max()) <= 0.02 * 3.47


def test_uniform_and_randint_ranges():
    u = synth.uniform01(synth.seed_of(9), (10000,))
    assert float(u.min()) >= 0.0 and float(u.max()) < 1.0
    r = synth.randint(synth.seed_of(9), (10000,), 1023)
    assert int(r.min()) >= 0 and int(r.max()) < 1023


def test_permutation_is_a_permutation():
    p = synth.permutation(synth.seed_of(3), 1000)
    assert sorted(p.tolist()) == list(range(1000))


def test_initial_tokens_layout():
    d = workloads.TINY
    t = workloads.initial_tokens(d)
    assert t.shape == (d.B, d.S) and t.dtype == torch.int32
    assert bool((t[:, d.prompt:] == d.mask_id).all())
    assert int(t[:, :d.prompt].max()) < d.vocab - 1
