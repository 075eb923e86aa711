"""Pins for the oracle's transformer pieces (CPU only).

Each check is fixed by mathematics or by an independent library routine, not
by re-typing the oracle's own formula.
"""
import numpy as np
import pytest
import scipy.special
import torch

from oracle.transformer import attention_rows, rmsnorm, rope, silu

RNG = np.random.default_rng(1234)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal((7, 64)) * 3.0
    g = np.ones(64)
    y = rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rmsnorm(5.0 * x, g, 0.0), y, rtol=1e-13)
    # gains scale each column
    g2 = RNG.standard_normal(64)
    np.testing.assert_allclose(rmsnorm(x, g2, 0.0), y * g2, rtol=1e-13)


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((5, 48))
    g = RNG.standard_normal(48)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-5), want, rtol=1e-12, atol=1e-14)


def test_rope_identity_at_zero_and_norm_preserving():
    x = RNG.standard_normal((3, 2, 16))
    np.testing.assert_array_equal(rope(x, np.zeros(3), 1e4), x)
    y = rope(x, np.array([1, 17, 4095]), 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_is_complex_rotation_in_pairs():
    # With D = 2 the pair (x0, x1) is the complex number x0 + i x1 rotated by pos * base^0 = pos.
    x = RNG.standard_normal((5, 1, 2))
    pos = np.array([0, 1, 2, 10, 100])
    y = rope(x, pos, 1e4)
    zc = (x[:, 0, 0] + 1j * x[:, 0, 1]) * np.exp(1j * pos)
    np.testing.assert_allclose(y[:, 0, 0], zc.real, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(y[:, 0, 1], zc.imag, rtol=1e-12, atol=1e-13)
    # second frequency of D = 4 rotates by pos * base^(-1/2)
    x4 = RNG.standard_normal((1, 1, 4))
    y4 = rope(x4, np.array([7]), 100.0)
    z2 = (x4[0, 0, 1] + 1j * x4[0, 0, 3]) * np.exp(1j * 7 * 100.0 ** -0.5)
    np.testing.assert_allclose([y4[0, 0, 1], y4[0, 0, 3]], [z2.real, z2.imag], rtol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    q = RNG.standard_normal((1, 1, 32))
    k = RNG.standard_normal((1, 1, 32))
    def score(m, n):
        return float(np.sum(rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4)))
    assert score(10, 3) == pytest.approx(score(107, 100), rel=1e-10)
    assert score(0, 0) == pytest.approx(float(np.sum(q * k)), rel=1e-12)


def test_silu():
    assert silu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-50, 50, 1001)
    np.testing.assert_allclose(silu(x), x * scipy.special.expit(x), rtol=1e-13, atol=1e-300)


def _sdpa(q, k, v):
    """torch's scaled_dot_product_attention (no mask) per query head, fp64 on the CPU."""
    R, Hq, D = q.shape
    g = Hq // k.shape[1]
    out = np.empty_like(q)
    for h in range(Hq):
        qt = torch.from_numpy(np.ascontiguousarray(q[:, h, :]))[None, None]
        kt = torch.from_numpy(np.ascontiguousarray(k[:, h // g, :]))[None, None]
        vt = torch.from_numpy(np.ascontiguousarray(v[:, h // g, :]))[None, None]
        out[:, h, :] = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
    return out


@pytest.mark.parametrize("R,S,Hq,Hkv,D", [(3, 5, 2, 2, 8), (4, 9, 4, 1, 16), (6, 33, 6, 2, 4)])
def test_attention_matches_torch_sdpa(R, S, Hq, Hkv, D):
    q = RNG.standard_normal((R, Hq, D))
    k = RNG.standard_normal((S, Hkv, D))
    v = RNG.standard_normal((S, Hkv, D))
    np.testing.assert_allclose(attention_rows(q, k, v), _sdpa(q, k, v), rtol=1e-11, atol=1e-12)


def test_attention_closed_forms():
    q = RNG.standard_normal((4, 2, 8))
    v = RNG.standard_normal((6, 2, 8))
    # one key: output is that value row
    np.testing.assert_allclose(attention_rows(q, RNG.standard_normal((1, 2, 8)), v[:1]), np.broadcast_to(v[:1], (4, 2, 8)), rtol=1e-14)
    # all keys equal: uniform weights, output is the mean of V
    k_eq = np.broadcast_to(RNG.standard_normal((1, 2, 8)), (6, 2, 8)).copy()
    np.testing.assert_allclose(attention_rows(q, k_eq, v), np.broadcast_to(v.mean(axis=0), (4, 2, 8)), rtol=1e-12)
    # non-causal: permuting cache rows leaves the output unchanged
    k = RNG.standard_normal((6, 2, 8))
    perm = RNG.permutation(6)
    np.testing.assert_allclose(attention_rows(q, k[perm], v[perm]), attention_rows(q, k, v), rtol=1e-12)
    # one key scored far above the rest selects its value row
    k2 = RNG.standard_normal((6, 2, 8)) * 1e-3
    k2[3] = q[0] * 1e3
    out = attention_rows(q[:1], k2, v)
    np.testing.assert_allclose(out[0], v[3], rtol=1e-9)


def test_gqa_equals_mha_with_repeated_kv():
    q = RNG.standard_normal((3, 4, 8))
    k = RNG.standard_normal((5, 2, 8))
    v = RNG.standard_normal((5, 2, 8))
    k_rep = np.repeat(k, 2, axis=1)
    v_rep = np.repeat(v, 2, axis=1)
    np.testing.assert_allclose(attention_rows(q, k, v), attention_rows(q, k_rep, v_rep), rtol=1e-14)


def test_bf16_softmax_weights_pins():
    """bf16 storage mode rounds the softmax weights that multiply V (the GPU's matrix-core operand)
    against a power-of-two reference.  Pins: (1) an exact rounding is the plain softmax; (2) when
    every weight 2^(x_j - M) is a power of two it is exact in bf16, so the result is the plain
    softmax; (3) the error is within the rounding bound 2^-9 sum_j p_j |V_j| (RNE to 8 significant
    bits); (4) shifting all scores of a query by an integer number of log2 units changes nothing,
    (5) a half-unit shift does change the rounded weights (the reference is an integer, not the
    row maximum itself)."""
    from oracle.numerics import round_bf16
    R, S, H, D = 3, 40, 2, 16
    q = RNG.standard_normal((R, H, D))
    k = RNG.standard_normal((S, H, D))
    v = RNG.standard_normal((S, H, D))
    exact = attention_rows(q, k, v)
    np.testing.assert_allclose(attention_rows(q, k, v, p_store=lambda w: w), exact, rtol=1e-12, atol=1e-13)
    # (2) scores s_j = n_j ln2: weights 2^(n_j - max n) are exact in bf16
    qd = np.zeros((1, 1, D))
    qd[0, 0, 0] = np.sqrt(D)            # s_j = k_j[0] with the 1/sqrt(D) scale
    kd = np.zeros((S, 1, D))
    kd[:, 0, 0] = RNG.integers(-6, 3, S) * np.log(2.0)
    vd = RNG.standard_normal((S, 1, D))
    np.testing.assert_allclose(attention_rows(qd, kd, vd, p_store=round_bf16), attention_rows(qd, kd, vd),
                               rtol=1e-12, atol=1e-13)
    # (3) the rounding bound
    got = attention_rows(q, k, v, p_store=round_bf16)
    a = attention_rows(q, k, np.abs(v))
    assert np.all(np.abs(got - exact) <= 2.0 ** -9 * a + 1e-12)
    assert np.max(np.abs(got - exact)) > 0          # the weights really are rounded
    # (4), (5): add t u to every key, u = q / |q|^2, so every score of that query rises by t / sqrt(D)
    for shift, same in ((3.0, True), (0.5, False)):
        q1 = q[:1, :1]
        u = q1[0, 0] / float(q1[0, 0] @ q1[0, 0])
        t = shift * np.log(2.0) * np.sqrt(D)
        k1 = k[:, :1] + t * u
        a0 = attention_rows(q1, k[:, :1], v[:, :1], p_store=round_bf16)
        a1 = attention_rows(q1, k1, v[:, :1], p_store=round_bf16)
        if same:
            np.testing.assert_allclose(a1, a0, rtol=1e-12, atol=1e-13)
        else:
            assert np.max(np.abs(a1 - a0)) > 1e-6
