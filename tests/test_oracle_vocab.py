"""Pins for confidence / argmax / local KL (CPU only)."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle.vocab import conf_kl, conf_kl_row

RNG = np.random.default_rng(11)


def test_uniform_logits():
    V = 1024
    z = np.full(V, 0.7)
    conf, arg, kl = conf_kl_row(z, z.copy(), exclude_id=V - 1)
    assert conf == pytest.approx(1.0 / (V - 1), rel=1e-14)
    assert arg == 0
    assert kl == 0.0
    conf2, arg2, _ = conf_kl_row(z, None, exclude_id=-1)
    assert conf2 == pytest.approx(1.0 / V, rel=1e-14) and arg2 == 0


def test_two_token_closed_form():
    for a, b in [(0.3, -1.2), (5.0, 5.0), (-2.0, 4.0)]:
        p = scipy.special.expit(a - b)
        for c, d in [(0.0, 0.0), (1.0, -1.0), (-3.0, 0.5)]:
            q = scipy.special.expit(c - d)
            conf, arg, kl = conf_kl_row(np.array([a, b]), np.array([c, d]))
            want = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
            assert kl == pytest.approx(want, rel=1e-10, abs=1e-15)
            assert conf == pytest.approx(max(p, 1 - p), rel=1e-14)
            assert arg == (0 if a >= b else 1)


def test_kl_matches_scipy_entropy_and_is_nonnegative():
    for _ in range(20):
        V = int(RNG.integers(3, 300))
        z = RNG.standard_normal(V) * 3
        zp = z + RNG.standard_normal(V) * 0.5
        _, _, kl = conf_kl_row(z, zp)
        want = scipy.stats.entropy(scipy.special.softmax(z), scipy.special.softmax(zp))
        assert kl == pytest.approx(want, rel=1e-9, abs=1e-14)
        assert kl >= 0.0


def test_exclusion_and_shift_invariance():
    V = 50
    z = RNG.standard_normal(V)
    z[V - 1] = 100.0                        # the excluded id would dominate
    zp = RNG.standard_normal(V)
    conf, arg, kl = conf_kl_row(z, zp, exclude_id=V - 1)
    assert arg != V - 1
    want = scipy.stats.entropy(scipy.special.softmax(z[:-1]), scipy.special.softmax(zp[:-1]))
    assert kl == pytest.approx(want, rel=1e-9)
    assert conf == pytest.approx(scipy.special.softmax(z[:-1]).max(), rel=1e-12)
    c2, a2, k2 = conf_kl_row(z + 37.0, zp - 11.0, exclude_id=V - 1)
    assert c2 == pytest.approx(conf, rel=1e-12) and a2 == arg and k2 == pytest.approx(kl, rel=1e-8, abs=1e-13)


def test_argmax_ties_to_lowest_id():
    z = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    assert conf_kl_row(z, None)[1] == 1
    assert conf_kl_row(z, None, exclude_id=1)[1] == 3


def test_identical_logits_kl_exactly_zero_batch():
    z = RNG.standard_normal((6, 200)) * 4
    conf, arg, kl = conf_kl(z, z.copy(), exclude_id=199)
    assert np.all(kl == 0.0)
    _, _, kl_none = conf_kl(z, None)
    assert np.all(np.isinf(kl_none))


# ---- compact KL state: previous logits kept in bf16 -------------------------------------------

def _bf16_grid(x):
    from oracle.numerics import round_bf16
    return round_bf16(x)


def test_bf16_state_identical_logits_give_zero_kl():
    """The state holds bf16(z); the next pass over the same fp32 logits compares bf16(z) with it: 0."""
    from oracle.vocab import kl_state_value
    for V in (2, 17, 1000):
        z = RNG.normal(0, 3, V).astype(np.float32).astype(np.float64)
        state = kl_state_value(z, prev_bf16=True)
        _, _, kl = conf_kl_row(z, state, exclude_id=V // 2 if V > 2 else -1, prev_bf16=True)
        assert kl == 0.0


def test_bf16_state_reduces_to_fp32_path_on_bf16_logits():
    """When every logit is a bf16 value the rounding is the identity: both state precisions agree exactly."""
    for _ in range(5):
        V = int(RNG.integers(2, 600))
        z = _bf16_grid(RNG.normal(0, 2, V))
        zp = _bf16_grid(RNG.normal(0, 2, V))
        a = conf_kl_row(z, zp, exclude_id=-1, prev_bf16=False)
        b = conf_kl_row(z, zp, exclude_id=-1, prev_bf16=True)
        assert a == b


def test_bf16_state_kl_matches_scipy_on_rounded_logits():
    """KL(softmax(bf16(z)) || softmax(z')) computed by scipy's relative entropy; conf/argmax unrounded."""
    for _ in range(5):
        V = int(RNG.integers(3, 800))
        z = RNG.normal(0, 2, V)
        zp = _bf16_grid(RNG.normal(0, 2, V))
        excl = int(RNG.integers(0, V))
        conf, arg, kl = conf_kl_row(z, zp, exclude_id=excl, prev_bf16=True)
        keep = np.arange(V) != excl
        p = scipy.special.softmax(_bf16_grid(z[keep]))
        q = scipy.special.softmax(zp[keep])
        assert kl == pytest.approx(scipy.stats.entropy(p, q), rel=1e-9, abs=1e-13)
        conf32, arg32, _ = conf_kl_row(z, zp, exclude_id=excl, prev_bf16=False)
        assert conf == conf32 and arg == arg32


def test_bf16_state_value_is_rne_rounding():
    from oracle.vocab import kl_state_value
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (bf16 spacing at 1): rounds to even (1.0)
    z = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0])
    assert kl_state_value(z, prev_bf16=True).tolist() == [1.0, 1.0 + 2.0 ** -6, -2.5, 0.0]
    assert kl_state_value(z, prev_bf16=False).tolist() == z.tolist()
