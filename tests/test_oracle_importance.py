"""Pins for the importance score (ES-dLLM Eq. 1 and its variants), CPU only."""
import numpy as np
import pytest
import scipy.spatial.distance

from oracle.importance import (FLT_MAX, VAR_COS, VAR_KL, VAR_L1N, VAR_L2REL, VAR_NONE,
                               importance_score, psi)

RNG = np.random.default_rng(7)


@pytest.mark.parametrize("var", [VAR_L1N, VAR_COS, VAR_L2REL])
def test_identical_rows_give_exactly_zero(var):
    h = RNG.standard_normal(4096)
    assert psi(h, h.copy(), var) == 0.0


def test_l1n_closed_form_single_spike():
    d = 256
    hp = np.ones(d)
    for delta in (1e-3, -0.5, 7.0):
        hc = hp.copy()
        hc[17] += delta
        # sum|dH| = |delta|, sqrt(d) * ||1||_2 = d
        assert psi(hc, hp, VAR_L1N) == pytest.approx(abs(delta) / d, rel=1e-14)


def test_l1n_scale_of_previous_row():
    hp = RNG.standard_normal(64)
    # H_cur = 2 H_prev: L1 change = sum|H_prev|, L2 relative change = 1, cosine change = 0
    assert psi(2 * hp, hp, VAR_L1N) == pytest.approx(np.abs(hp).sum() / (8.0 * np.linalg.norm(hp)), rel=1e-14)
    assert psi(2 * hp, hp, VAR_L2REL) == pytest.approx(1.0, rel=1e-14)
    assert psi(2 * hp, hp, VAR_COS) == pytest.approx(0.0, abs=1e-15)


def test_cosine_change_closed_forms_and_library():
    e0 = np.zeros(8); e0[0] = 1.0
    e1 = np.zeros(8); e1[1] = 3.0
    assert psi(e0, e1, VAR_COS) == pytest.approx(1.0, rel=1e-15)       # orthogonal
    assert psi(-2 * e0, e0, VAR_COS) == pytest.approx(2.0, rel=1e-15)  # antiparallel
    for _ in range(20):
        a = RNG.standard_normal(300)
        b = a + RNG.standard_normal(300) * 0.3
        # scipy's cosine distance is 1 - cos
        assert psi(a, b, VAR_COS) == pytest.approx(scipy.spatial.distance.cosine(a, b), rel=1e-10)


def test_zero_norm_rows():
    z = np.zeros(16)
    h = RNG.standard_normal(16)
    for var in (VAR_L1N, VAR_L2REL, VAR_COS):
        assert psi(z, z, var) == 0.0
        assert psi(h, z, var) == FLT_MAX
    assert psi(z, h, VAR_COS) == FLT_MAX
    assert psi(z, h, VAR_L2REL) == pytest.approx(1.0)


def test_score_combination():
    N, w = 12, 32
    hc = RNG.standard_normal((N, w))
    hp = hc + RNG.standard_normal((N, w)) * 0.1
    conf = RNG.uniform(size=N).astype(np.float32).astype(np.float64)
    kl = RNG.uniform(size=N)
    # alpha = 1 reproduces the (fp32) confidence bit for bit, or 1 - c when inverted
    s1 = importance_score(hc, hp, conf, kl, alpha=1.0, var=VAR_L1N, conf_inverted=False)
    np.testing.assert_array_equal(s1, conf)
    s1i = importance_score(hc, hp, conf, kl, alpha=1.0, var=VAR_NONE, conf_inverted=True)
    np.testing.assert_array_equal(s1i, (1.0 - conf).astype(np.float32).astype(np.float64))
    # alpha = 0 is the change term alone; the KL variant reads kl_prev
    s0 = importance_score(hc, hp, conf, kl, alpha=0.0, var=VAR_KL, conf_inverted=False)
    np.testing.assert_array_equal(s0, kl.astype(np.float32).astype(np.float64))
    # scores are fp32 values
    s = importance_score(hc, hp, conf, kl, alpha=0.5, var=VAR_COS, conf_inverted=True)
    np.testing.assert_array_equal(s, s.astype(np.float32).astype(np.float64))
    # a larger change of the hidden state never lowers the score (equal confidence)
    hp2 = hc.copy(); hp2[0] += 0.01; hp2[1] += 0.5
    s2 = importance_score(hc, hp2, np.full(N, 0.3), None, alpha=0.5, var=VAR_L1N, conf_inverted=False)
    assert s2[1] > s2[0] > s2[2] == pytest.approx(0.15)
