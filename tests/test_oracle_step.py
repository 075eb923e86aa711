"""Whole-iteration pins of the oracle (CPU only, exact float64 mode).

P1  with every row active, the partial update equals dense recompute;
P2  skipped rows keep their cached K/V, final hidden state and statistics bit for bit;
P5  if nothing changed since the cache was filled, active rows equal dense recompute;
P6  the LM head on every row of the final hidden state reproduces the cached statistics;
plus SureLock locking (locked rows are never recomputed yet stay attended).
"""
import numpy as np
import pytest

from oracle import dense_forward, lm_logits, conf_kl, layer_rows
from oracle.importance import VAR_COS, VAR_L1N
from oracle.step import (SEL_THRESH_CAP, SEL_TOPK, SEL_UNLOCKED, OracleModel, ScoreCfg,
                         StepCfg, new_state, skip_step)

L, d, Hq, Hkv, D, F, V, B, S = 3, 32, 4, 2, 8, 48, 41, 2, 12
MASK = V - 1


def tiny_model(seed=0, mode="exact"):
    rng = np.random.default_rng(seed)
    def w(*shape, std=0.3):
        return rng.standard_normal(shape) * std
    layers = []
    for _ in range(L):
        layers.append({"attn_norm": 1.0 + 0.1 * w(d), "wq": w(Hq * D, d), "wk": w(Hkv * D, d),
                       "wv": w(Hkv * D, d), "wo": w(d, Hq * D), "ffn_norm": 1.0 + 0.1 * w(d),
                       "wg": w(F, d), "wu": w(F, d), "wd": w(d, F)})
    weights = {"embed": w(V, d, std=1.0), "layers": layers, "final_norm": 1.0 + 0.1 * w(d), "lm_head": w(V, d)}
    return OracleModel(weights, Hq, Hkv, MASK, mode=mode)


def tokens(seed=1, n_prompt=6):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, V - 1, (B, S))
    t[:, n_prompt:] = MASK
    return t


def dense(model, tok, b=None):
    return dense_forward(model.weights, tok, n_heads=Hq, n_kv_heads=Hkv, rope_base=model.rope_base,
                         eps=model.eps, store=lambda v: v, boundary_layer=b)


def full_step(model, tok, b, track_kl=True):
    st = new_state(model, tok, track_kl)
    return skip_step(model, st, StepCfg(boundary_layer=b, full_step=True))


def test_full_step_equals_dense():
    m = tiny_model()
    tok = tokens()
    st, _ = full_step(m, tok, 1)
    ref = dense(m, tok, 1)
    for l in range(L):
        np.testing.assert_allclose(st.k_cache[l], ref["k"][l], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st.v_cache[l], ref["v"][l], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.h_fin, ref["h_fin"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.h_bnd_prev, ref["h_bnd"], rtol=1e-12, atol=1e-12)
    conf, arg, _ = conf_kl(ref["logits"].reshape(B * S, V), None, MASK)
    np.testing.assert_allclose(st.conf.reshape(-1), conf, rtol=1e-12)
    np.testing.assert_array_equal(st.argmax.reshape(-1), arg)


@pytest.mark.parametrize("b", [0, 1, 3])
def test_p1_all_rows_active_equals_dense(b):
    m = tiny_model(3)
    tok0 = tokens(4)
    st, _ = full_step(m, tok0, b)
    tok1 = tok0.copy()
    tok1[:, 7] = 5                     # the input changed since the cache was filled
    st.tokens = tok1
    cfg = StepCfg(boundary_layer=b, full_step=False, score=ScoreCfg(alpha=0.5, var=VAR_L1N, k=S))
    st2, info = skip_step(m, st, cfg)
    assert len(info["rows"]) == B * S
    ref = dense(m, tok1, b)
    np.testing.assert_allclose(st2.h_fin, ref["h_fin"], rtol=1e-11, atol=1e-11)
    for l in range(L):
        np.testing.assert_allclose(st2.k_cache[l], ref["k"][l], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(info["logits"], ref["logits"].reshape(B * S, V), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("b", [0, 2])
def test_p2_skipped_rows_bytes_unchanged(b):
    m = tiny_model(5)
    tok0 = tokens(6)
    st, _ = full_step(m, tok0, b)
    st.tokens[:, 8] = 3
    k = 4
    cfg = StepCfg(boundary_layer=b, full_step=False, score=ScoreCfg(alpha=0.5, var=VAR_COS, conf_inverted=True, k=k))
    st2, info = skip_step(m, st, cfg)
    rows = info["rows"]
    assert len(rows) == B * k
    skipped = np.setdiff1d(np.arange(B * S), rows)
    for l in range(b, L):
        for before, after in ((st.k_cache[l], st2.k_cache[l]), (st.v_cache[l], st2.v_cache[l])):
            fb = before.reshape(B * S, -1)
            fa = after.reshape(B * S, -1)
            assert np.array_equal(fb[skipped], fa[skipped])
            assert not np.array_equal(fb[rows], fa[rows])
    for name in ("h_fin", "conf", "kl", "argmax"):
        fb = getattr(st, name).reshape(B * S, -1)
        fa = getattr(st2, name).reshape(B * S, -1)
        assert np.array_equal(fb[skipped], fa[skipped]), name
    assert np.array_equal(st.logits_prev[skipped], st2.logits_prev[skipped])
    # layers below the boundary were recomputed on every row
    if b > 0:
        assert not np.array_equal(st.k_cache[0], st2.k_cache[0])


def test_p5_unchanged_input_sparse_equals_dense_on_active_rows():
    m = tiny_model(7)
    tok = tokens(8)
    st, _ = full_step(m, tok, 1)
    cfg = StepCfg(boundary_layer=1, full_step=False, score=ScoreCfg(alpha=0.3, var=VAR_L1N, k=5))
    st2, info = skip_step(m, st, cfg)
    ref = dense(m, tok, 1)
    rows = info["rows"]
    np.testing.assert_allclose(st2.h_fin.reshape(B * S, d)[rows], ref["h_fin"].reshape(B * S, d)[rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(info["logits"], ref["logits"].reshape(B * S, V)[rows], rtol=1e-10, atol=1e-11)
    # the importance change term is zero on every row: the ranking follows confidence
    np.testing.assert_allclose(info["scores"], 0.3 * st.conf.astype(np.float32), rtol=1e-6)


def test_p6_lm_head_on_all_rows_reproduces_statistics():
    m = tiny_model(9)
    tok = tokens(10)
    st, _ = full_step(m, tok, 2)
    st.tokens[:, 9] = 1
    st2, info = skip_step(m, st, StepCfg(boundary_layer=2, full_step=False, score=ScoreCfg(k=3)))
    z = lm_logits(st2.h_fin.reshape(B * S, d), m.weights["final_norm"], m.weights["lm_head"], m.eps, lambda v: v)
    conf, arg, _ = conf_kl(z, None, MASK)
    np.testing.assert_allclose(conf, st2.conf.reshape(-1), rtol=1e-13)
    np.testing.assert_array_equal(arg, st2.argmax.reshape(-1))
    np.testing.assert_allclose(z, st2.logits_prev, rtol=1e-13)


def test_kl_zero_when_input_unchanged_and_lock():
    m = tiny_model(11)
    tok = tokens(12)
    st, _ = full_step(m, tok, 0)
    assert np.all(np.isinf(st.kl))
    cfg = StepCfg(boundary_layer=0, full_step=False, score=ScoreCfg(sel=SEL_UNLOCKED, alpha=0.0, var=VAR_L1N),
                  lock_kl_eps=1e-12, lock_conf_min=-1.0)
    st2, info = skip_step(m, st, cfg)
    # same tokens, every row recomputed: every posterior is identical, KL = 0, all rows lock
    np.testing.assert_allclose(st2.kl, 0.0, atol=1e-12)
    assert np.all(st2.force == 2)


def test_locked_rows_skip_compute_but_stay_attended():
    m = tiny_model(13)
    tok = tokens(14)
    st, _ = full_step(m, tok, 0)
    st.force[:, :4] = 2                     # lock the first four positions of each sequence
    st.tokens[:, 10] = 2                     # change the input of an unlocked position
    cfg = StepCfg(boundary_layer=0, full_step=False, score=ScoreCfg(sel=SEL_UNLOCKED))
    st2, info = skip_step(m, st, cfg)
    rows = info["rows"]
    assert len(rows) == B * (S - 4) and np.all(rows % S >= 4)
    for l in range(L):
        assert np.array_equal(st.k_cache[l][:, :4], st2.k_cache[l][:, :4])
    # reference: attention of the active rows over cache rows whose first four positions
    # hold the K/V computed when the rows were last run
    x = m.weights["embed"][st.tokens.reshape(-1)][rows]
    kc = [k.copy() for k in st.k_cache]
    vc = [v.copy() for v in st.v_cache]
    for l in range(L):
        x = layer_rows(m.weights["layers"][l], x, rows % S, rows // S, kc[l], vc[l], n_heads=Hq,
                       n_kv_heads=Hkv, rope_base=m.rope_base, eps=m.eps, store=lambda v: v)
    np.testing.assert_allclose(st2.h_fin.reshape(B * S, d)[rows], x, rtol=1e-13)
    # and this differs from a dense recompute (the locked rows' stale K/V matter)
    ref = dense(m, st.tokens)
    assert not np.allclose(st2.h_fin.reshape(B * S, d)[rows], ref["h_fin"].reshape(B * S, d)[rows], rtol=1e-9)


def test_thresh_cap_step_and_unmask():
    m = tiny_model(15)
    tok = tokens(16)
    st, _ = full_step(m, tok, 1)
    st.force[:, :6] = 2                       # prompt rows excluded
    st.force[:, 8] = 1                        # forced row
    st.tokens[:, 7] = 4
    cfg = StepCfg(boundary_layer=1, full_step=False,
                  score=ScoreCfg(alpha=0.0, var=VAR_COS, sel=SEL_THRESH_CAP, tau=1e-3, k=3),
                  unmask_n=2, block_lo=6, block_hi=12)
    st2, info = skip_step(m, st, cfg)
    rows = info["rows"]
    for bb in range(B):
        r = rows[rows // S == bb] % S
        assert 8 in r and len(r) <= 3 and np.all(r >= 6)
    # unmask picked the two most confident masked positions of the block
    for bb in range(B):
        changed = np.nonzero(st2.tokens[bb] != st.tokens[bb])[0]
        assert len(changed) == 2 and np.all((changed >= 6) & (changed < 12))
        masked = [i for i in range(6, 12) if st.tokens[bb, i] == MASK]
        order = sorted(masked, key=lambda i: (-st2.conf[bb, i], i))
        assert sorted(order[:2]) == changed.tolist()


def test_bf16_mode_close_to_exact():
    me = tiny_model(17, "exact")
    mb = tiny_model(17, "bf16")
    from oracle.numerics import round_bf16
    for mm in (me, mb):   # bf16-valued weights for both
        mm.weights["embed"] = round_bf16(mm.weights["embed"])
    tok = tokens(18)
    se, _ = full_step(me, tok, 1)
    sb, _ = full_step(mb, tok, 1)
    err = np.abs(sb.h_fin - se.h_fin).max() / np.abs(se.h_fin).max()
    # bf16 mode rounds at 10 storage points per layer (two RMSNorm outputs, Q, K, V, the softmax
    # weights, the attention output, the residual stream twice, SwiGLU): 30 roundings of relative
    # size <= 2^-9 over these 3 layers (the distance is about 1.6e-2 without and 2.0e-2 with the
    # softmax weights rounded)
    assert 0 < err < 30 * 2.0 ** -9


# ---- nested boundaries: later layers narrow the active set (ES-dLLM 2.1 item 2, I_{l,i}) -------

def test_nested_full_step_fills_cache_with_layer_input():
    """A full step stores, for every row, the hidden state entering each nested layer (= dense pass)."""
    m = tiny_model(21)
    tok = tokens(22)
    st = new_state(m, tok, True, n_nested=2)
    st2, _ = skip_step(m, st, StepCfg(boundary_layer=0, full_step=True, nested=((1, 3), (2, 2))))
    for j, nl in enumerate((1, 2)):
        np.testing.assert_allclose(st2.h_nested[j], dense(m, tok, nl)["h_bnd"], rtol=1e-12, atol=1e-12)


def test_nested_keeping_every_row_equals_single_boundary():
    m = tiny_model(23)
    tok = tokens(24)
    st = new_state(m, tok, True, n_nested=1)
    st, _ = skip_step(m, st, StepCfg(boundary_layer=1, full_step=True, nested=((2, 5),)))
    st.tokens[:, 9] = 4
    sc = ScoreCfg(alpha=0.5, var=VAR_L1N, k=5)
    a, ia = skip_step(m, st, StepCfg(boundary_layer=1, full_step=False, score=sc))
    b, ib = skip_step(m, st, StepCfg(boundary_layer=1, full_step=False, score=sc, nested=((2, 5),)))
    assert np.array_equal(ia["rows"], ib["rows"]) and np.array_equal(ib["nested_rows"][0], ib["rows"])
    for name in ("h_fin", "conf", "kl", "argmax"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    for l in range(L):
        assert np.array_equal(a.k_cache[l], b.k_cache[l]) and np.array_equal(a.v_cache[l], b.v_cache[l])


def test_nested_unchanged_input_selects_by_confidence():
    """Nothing changed since the caches were filled: every change term is 0 (P5), so each nested
    stage keeps the k most confident rows of the previous stage (ties to the lower position),
    checked here by a brute-force ordering."""
    m = tiny_model(25)
    tok = tokens(26)
    st = new_state(m, tok, True, n_nested=2)
    st, _ = skip_step(m, st, StepCfg(boundary_layer=0, full_step=True, nested=((1, 8), (2, 3))))
    alpha = 0.7
    cfg = StepCfg(boundary_layer=0, full_step=False, score=ScoreCfg(alpha=alpha, var=VAR_COS, k=8),
                  nested=((1, 5), (2, 3)))
    st2, info = skip_step(m, st, cfg)
    conf = st.conf.reshape(-1)
    prev = info["nested_rows"][0]
    stages = [np.concatenate([b * S + np.array(sorted(sorted(range(S), key=lambda i: (-conf[b * S + i], i))[:8]))
                              for b in range(B)])]
    for k in (5, 3):
        keep = []
        for b in range(B):
            cand = [r for r in stages[-1] if r // S == b]
            keep += sorted(sorted(cand, key=lambda r: (-np.float32(alpha * conf[r]), r))[:k])
        stages.append(np.array(keep))
    assert np.array_equal(prev, stages[1])
    assert np.array_equal(info["nested_rows"][1], stages[2])
    assert np.array_equal(info["rows"], stages[2])


def test_nested_dropped_rows_are_skipped_from_their_layer_on():
    m = tiny_model(27)
    tok = tokens(28)
    st = new_state(m, tok, True, n_nested=1)
    st, _ = skip_step(m, st, StepCfg(boundary_layer=0, full_step=True, nested=((2, 4),)))
    st.tokens[:, 7] = 2
    st.tokens[:, 10] = 3
    cfg = StepCfg(boundary_layer=0, full_step=False, score=ScoreCfg(alpha=0.5, var=VAR_L1N, k=7), nested=((2, 3),))
    st2, info = skip_step(m, st, cfg)
    before = info["nested_rows"][0]
    final = info["rows"]
    assert np.array_equal(before, final) and len(final) == B * 3
    # rows that reached layer 2 (the boundary selection) vs the ones that continued past it
    reached = np.nonzero(np.any(st2.h_nested[0].reshape(B * S, d) != st.h_nested[0].reshape(B * S, d), axis=1))[0]
    assert set(final) <= set(reached) and len(reached) == B * 7
    dropped = np.setdiff1d(reached, final)
    for name in ("h_fin", "conf", "kl", "argmax"):
        fb = getattr(st, name).reshape(B * S, -1)
        fa = getattr(st2, name).reshape(B * S, -1)
        assert np.array_equal(fb[dropped], fa[dropped]), name
        assert not np.array_equal(fb[final], fa[final]), name
    for l in range(L):
        kb, ka = st.k_cache[l].reshape(B * S, -1), st2.k_cache[l].reshape(B * S, -1)
        if l == 1:  # layer 1 ran on every row selected at the boundary, and attention mixed in the change
            assert not np.any(np.all(kb[dropped] == ka[dropped], axis=1))
        elif l >= 2:  # from layer 2 on the dropped rows are skipped
            assert np.array_equal(kb[dropped], ka[dropped])


@pytest.mark.parametrize("nested", [((0, 2),), ((2, 2), (2, 1)), ((3, 2),), ((2, -1),)])
def test_nested_layers_validated(nested):
    m = tiny_model(29)
    tok = tokens(30)
    st = new_state(m, tok, True, n_nested=2)
    with pytest.raises(ValueError):
        skip_step(m, st, StepCfg(boundary_layer=0, full_step=True, nested=nested))


# ---- per-layer cache (dLLM-Cache summary section 3) ----

def _lc_full(m, tok, b):
    st = new_state(m, tok, True, layer_cache=True)
    return skip_step(m, st, StepCfg(boundary_layer=b, full_step=True, layer_cache=True))


@pytest.mark.parametrize("b", [0, 1])
def test_layer_cache_full_step_fills_caches_with_dense_layer_io(b):
    """Full step: the cache of layer l >= b holds the dense pass's hidden state entering layer l
    (input) and entering layer l + 1 (output; the final hidden state after the last layer)."""
    m = tiny_model(21)
    tok = tokens(22)
    st, _ = _lc_full(m, tok, b)
    for l in range(L):
        if l < b:
            assert not st.x_in[l].any() and not st.x_out[l].any()
            continue
        np.testing.assert_allclose(st.x_in[l], dense(m, tok, l)["h_bnd"], rtol=1e-12, atol=1e-12)
        want_out = dense(m, tok, l + 1)["h_bnd"] if l + 1 < L else dense(m, tok)["h_fin"]
        np.testing.assert_allclose(st.x_out[l], want_out, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b", [0, 2])
def test_layer_cache_every_row_equals_dense(b):
    """k = S: every row recomputed at every layer, so the step is the dense recompute of the new
    tokens (K/V of every layer, final hidden state, logits)."""
    m = tiny_model(23)
    tok = tokens(24)
    st, _ = _lc_full(m, tok, b)
    st.tokens[0, 7] = 3
    st.tokens[1, 10] = 5
    st2, info = skip_step(m, st, StepCfg(boundary_layer=b, full_step=False, layer_cache=True,
                                         score=ScoreCfg(alpha=0.0, var=VAR_COS, k=S)))
    ref = dense(m, st.tokens)
    for l in range(L):
        np.testing.assert_allclose(st2.k_cache[l], ref["k"][l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(st2.v_cache[l], ref["v"][l], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st2.h_fin, ref["h_fin"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(info["logits"], ref["logits"].reshape(B * S, V), rtol=1e-10, atol=1e-11)
    assert len(info["layer_rows"]) == L - b


def test_layer_cache_unchanged_tokens_reproduce_dense_and_tie_on_index():
    """Nothing changed since the full step: every change term is 0, so each layer keeps the first
    k positions of every sequence, and reused and recomputed rows both equal the dense values."""
    m = tiny_model(25)
    tok = tokens(26)
    st, _ = _lc_full(m, tok, 0)
    k = 3
    st2, info = skip_step(m, st, StepCfg(boundary_layer=0, full_step=False, layer_cache=True,
                                         score=ScoreCfg(alpha=0.0, var=VAR_COS, k=k)))
    want = np.concatenate([bb * S + np.arange(k) for bb in range(B)])
    for sel in info["layer_rows"]:
        np.testing.assert_array_equal(sel, want)
    for sc in info["layer_scores"]:
        assert np.all(np.abs(sc) < 1e-12)
    ref = dense(m, tok)
    np.testing.assert_allclose(st2.h_fin, ref["h_fin"], rtol=1e-11, atol=1e-12)
    for l in range(L):
        np.testing.assert_allclose(st2.x_out[l], st.x_out[l], rtol=1e-11, atol=1e-12)


def test_layer_cache_selects_the_changed_row_and_reuses_the_rest():
    """One token changes: at layer 0 only its row's input differs from the cache, so with k = 1 and
    the cosine change term that row is recomputed; every other row keeps its cached layer output
    and K/V, and rows not recomputed at the last layer keep their statistics."""
    m = tiny_model(27)
    tok = tokens(28)
    st, _ = _lc_full(m, tok, 0)
    p = 8
    st.tokens[1, p] = 4
    st2, info = skip_step(m, st, StepCfg(boundary_layer=0, full_step=False, layer_cache=True,
                                         score=ScoreCfg(alpha=0.0, var=VAR_COS, k=1)))
    sel0 = info["layer_rows"][0]
    assert sel0[1] == S + p                                     # sequence 1: the changed position
    assert info["layer_scores"][0][1, p] > 0 and np.all(np.delete(info["layer_scores"][0][1], p) < 1e-12)
    others = np.setdiff1d(np.arange(B * S), sel0)
    np.testing.assert_array_equal(st2.x_out[0].reshape(B * S, d)[others], st.x_out[0].reshape(B * S, d)[others])
    kc0, kc1 = st.k_cache[0].reshape(B * S, -1), st2.k_cache[0].reshape(B * S, -1)
    np.testing.assert_array_equal(kc1[others], kc0[others])
    assert not np.allclose(kc1[S + p], kc0[S + p])
    np.testing.assert_array_equal(st2.x_in[0].reshape(B * S, d)[S + p], m.weights["embed"][4])
    last = info["rows"]
    keep = np.setdiff1d(np.arange(B * S), last)
    np.testing.assert_array_equal(st2.h_fin.reshape(B * S, d)[keep], st.h_fin.reshape(B * S, d)[keep])
    np.testing.assert_array_equal(st2.conf.reshape(-1)[keep], st.conf.reshape(-1)[keep])
    np.testing.assert_array_equal(st2.argmax.reshape(-1)[keep], st.argmax.reshape(-1)[keep])
    np.testing.assert_array_equal(st2.h_fin.reshape(B * S, d)[last], st2.x_out[L - 1].reshape(B * S, d)[last])


def test_layer_cache_locked_prompt_rows_are_never_recomputed():
    """Long-interval prompt cache: prompt positions locked (force 2) between full steps are never
    selected and keep their cached K/V at every layer."""
    m = tiny_model(29)
    tok = tokens(30)
    st, _ = _lc_full(m, tok, 0)
    st.force[:, :6] = 2
    st.tokens[0, 9] = 2
    st2, info = skip_step(m, st, StepCfg(boundary_layer=0, full_step=False, layer_cache=True,
                                         score=ScoreCfg(alpha=0.0, var=VAR_COS, k=4)))
    for sel in info["layer_rows"]:
        assert np.all(sel % S >= 6)
    for l in range(L):
        np.testing.assert_array_equal(st2.k_cache[l][:, :6], st.k_cache[l][:, :6])


def test_layer_cache_validated():
    m = tiny_model(31)
    tok = tokens(32)
    st = new_state(m, tok, True)                       # no per-layer caches
    with pytest.raises(ValueError):
        skip_step(m, st, StepCfg(boundary_layer=0, full_step=True, layer_cache=True))
    st, _ = _lc_full(m, tok, 0)
    with pytest.raises(ValueError):
        skip_step(m, st, StepCfg(boundary_layer=1, full_step=False, layer_cache=True, nested=((2, 1),)))


# ---- per-layer cache compared on V (dLLM-Cache summary section 3: feature-similarity test) ----

def _vc_step(m, st, b, k, sel=SEL_TOPK):
    return skip_step(m, st, StepCfg(boundary_layer=b, full_step=False, layer_cache=True, cache_feature="value",
                                    score=ScoreCfg(alpha=0.0, var=VAR_COS, sel=sel, k=k)))


@pytest.mark.parametrize("b", [0, 1])
def test_value_cache_every_row_equals_dense(b):
    """k = S with the V feature: every row recomputed at every layer, so the step is the dense
    recompute of the new tokens."""
    m = tiny_model(33)
    tok = tokens(34)
    st, _ = _lc_full(m, tok, b)
    st.tokens[0, 7] = 3
    st.tokens[1, 9] = 6
    st2, info = _vc_step(m, st, b, S)
    ref = dense(m, st.tokens)
    for l in range(L):
        np.testing.assert_allclose(st2.k_cache[l], ref["k"][l], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(st2.v_cache[l], ref["v"][l], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st2.h_fin, ref["h_fin"], rtol=1e-11, atol=1e-12)


def test_value_cache_unchanged_tokens_tie_on_index():
    """Nothing changed since the full step: every row's V equals its cached V exactly, so every
    change term is 0 and each layer keeps the first k positions; the state equals the dense pass."""
    m = tiny_model(35)
    tok = tokens(36)
    st, _ = _lc_full(m, tok, 0)
    k = 4
    st2, info = _vc_step(m, st, 0, k)
    want = np.concatenate([bb * S + np.arange(k) for bb in range(B)])
    for sel, sc in zip(info["layer_rows"], info["layer_scores"]):
        np.testing.assert_array_equal(sel, want)
        assert np.all(sc == 0.0)
    np.testing.assert_allclose(st2.h_fin, dense(m, tok)["h_fin"], rtol=1e-11, atol=1e-12)


def test_value_cache_selection_matches_brute_force_cosine():
    """Two tokens change.  Layer 0: only their rows' V differ from the cache, so they come first.
    Layer 1: every row's input differs (attention mixes the change in); the selected rows are the
    k with the largest cosine distance (scipy) between the V projection of the row's input --
    recomputed here from the layer's output cache -- and the V cached before the step; the locked
    prompt rows never compete."""
    from scipy.spatial.distance import cosine
    from oracle.transformer import rmsnorm
    m = tiny_model(37)
    tok = tokens(38)
    st, _ = _lc_full(m, tok, 0)
    st.force[:, :4] = 2
    st.tokens[0, 7] = 3
    st.tokens[1, 10] = 5
    k = 3
    st2, info = _vc_step(m, st, 0, k)
    sel0 = info["layer_rows"][0]
    assert {7, S + 10} <= set(sel0.tolist())
    lw = m.weights["layers"][1]
    x1 = st2.x_out[0].reshape(B * S, d)          # the input of layer 1 of every row after the step
    v_new = rmsnorm(x1, lw["attn_norm"], m.eps) @ lw["wv"].T
    v_old = st.v_cache[1].reshape(B * S, -1)
    for bb in range(B):
        dist = np.array([cosine(v_new[bb * S + i], v_old[bb * S + i]) for i in range(S)])
        dist[:4] = -np.inf                        # locked rows do not compete
        order = sorted(range(S), key=lambda i: (-dist[i], i))
        got = info["layer_rows"][1][info["layer_rows"][1] // S == bb] % S
        np.testing.assert_array_equal(got, np.sort(order[:k]))
        srt = np.sort(dist[4:])[::-1]
        assert srt[k - 1] - srt[k] > 1e-9         # no near tie at the boundary
    # the hidden-state feature ranks layer 1 differently on this input (the feature is really V)
    _, info_h = skip_step(m, st, StepCfg(boundary_layer=0, full_step=False, layer_cache=True,
                                         score=ScoreCfg(alpha=0.0, var=VAR_COS, k=k)))
    assert not np.allclose(info_h["layer_scores"][1], info["layer_scores"][1])


def test_value_cache_validated():
    m = tiny_model(39)
    tok = tokens(40)
    st, _ = _lc_full(m, tok, 0)
    with pytest.raises(ValueError):
        skip_step(m, st, StepCfg(boundary_layer=0, full_step=False, layer_cache=True, cache_feature="key",
                                 score=ScoreCfg(alpha=0.0, var=VAR_COS, k=2)))
