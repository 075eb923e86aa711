"""End-to-end parity of dllm_skip_step with the oracle's iteration (GPU)."""
import numpy as np
import pytest
import torch

import synth
from oracle.importance import VAR_COS, VAR_L1N
from oracle.selection import FORCE_EXCLUDED
from oracle.dus import dus_rounds
from oracle.step import (SEL_THRESH_CAP, SEL_TOPK, SEL_UNLOCKED, UNMASK_FORCED, OracleModel, ScoreCfg, StepCfg,
                         new_state, skip_step)
from synth import workloads
from tests.gpu_util import DEV, assert_close, assert_within, kl_first_order, np64, selection_gap
from tests.helpers import oracle_weights
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def _models(dims, std=workloads.WEIGHT_STD):
    w = workloads.model_weights(dims, std=std)
    wd = {"embed": w["embed"].to(DEV), "final_norm": w["final_norm"].to(DEV), "lm_head": w["lm_head"].to(DEV),
          "layers": [{k: t.to(DEV) for k, t in lw.items()} for lw in w["layers"]]}
    gm = api.Model(wd, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    om = OracleModel(oracle_weights(w), dims.n_heads, dims.n_kv_heads, dims.mask_id,
                     mode="exact" if dims.dtype == "f32" else "bf16")
    return gm, om


def _score_cfg_pair(alpha, var, sel, k, tau=0.0, conf_inverted=False):
    return (api.score_cfg(alpha=alpha, conf_inverted=conf_inverted, var=var, sel=sel, k=k, tau=tau),
            ScoreCfg(alpha=alpha, conf_inverted=conf_inverted, var=var, sel=sel, k=k, tau=tau))


def _compare_state(gs, os_, rows, tol, what, check_argmax_gap=True):
    B, S = os_.tokens.shape
    flat = np.asarray(rows)
    assert_close(np64(gs.h_fin).reshape(B * S, -1)[flat], os_.h_fin.reshape(B * S, -1)[flat], tol, f"{what} h_fin")
    assert_close(np64(gs.conf).reshape(-1)[flat], os_.conf.reshape(-1)[flat], max(tol, 1e-4), f"{what} conf")
    if gs.logits_prev is not None:
        assert_close(np64(gs.logits_prev)[flat], os_.logits_prev[flat], tol, f"{what} logits")


def _argmax_ok(gs, os_, rows, margin):
    """argmax must match wherever the oracle's top-2 logit gap exceeds `margin`."""
    if os_.logits_prev is None:
        return
    B, S = os_.tokens.shape
    ga = gs.argmax.cpu().numpy().reshape(-1)
    for r in rows:
        z = os_.logits_prev[r].copy()
        z[-1] = -np.inf
        top2 = np.sort(z)[-2:]
        if top2[1] - top2[0] > margin:
            assert ga[r] == os_.argmax.reshape(-1)[r], f"argmax row {r}"


def test_tiny_fp32_two_iterations():
    """The tiny fp32 workload: full iteration, unmask 4, then an early-skip iteration (top 25% after layer 0)."""
    dims = workloads.TINY
    gm, om = _models(dims)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=32, track_kl=True)
    ws = api.alloc_workspace(gm, dims.B, dims.S, 32)
    os_ = new_state(om, tok.numpy(), track_kl=True)
    lo, hi = dims.prompt, dims.S
    # iteration t-1: full
    api.skip_step(gm, gs, api.step_cfg(1, True, unmask_n=4, block_lo=lo, block_hi=hi, ws=ws))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=1, full_step=True, unmask_n=4, block_lo=lo, block_hi=hi))
    torch.cuda.synchronize()
    allrows = np.arange(dims.B * dims.S)
    _compare_state(gs, os_, allrows, 1e-4, "full")
    np.testing.assert_array_equal(gs.argmax.cpu().numpy(), os_.argmax)
    np.testing.assert_array_equal(gs.tokens.cpu().numpy(), os_.tokens)
    for l in range(dims.n_layers):
        assert_close(np64(gs.k_cache[l]), os_.k_cache[l], 1e-4, f"K cache {l}")
        assert_close(np64(gs.v_cache[l]), os_.v_cache[l], 1e-4, f"V cache {l}")
    # iteration t: layer 0 full, layer 1 on the top 25% by 0.5 (1 - conf) + 0.5 (1 - cos)
    gsc, osc = _score_cfg_pair(0.5, VAR_COS, SEL_TOPK, 32, conf_inverted=True)
    api.skip_step(gm, gs, api.step_cfg(1, False, gsc, unmask_n=4, block_lo=lo, block_hi=hi, ws=ws))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=1, full_step=False, score=osc, unmask_n=4,
                                           block_lo=lo, block_hi=hi))
    torch.cuda.synchronize()
    gap = selection_gap(info["scores"][0], None, 32)
    assert gap > 1e-6, f"near tie at the selection boundary ({gap})"
    idx = gs.idx.cpu().numpy()
    assert int(gs.n_active[0]) == 32
    np.testing.assert_array_equal(idx[0], info["rows"])
    _compare_state(gs, os_, info["rows"], 1e-4, "sparse")
    np.testing.assert_array_equal(gs.tokens.cpu().numpy(), os_.tokens)
    np.testing.assert_array_equal(gs.argmax.cpu().numpy(), os_.argmax)
    for l in range(dims.n_layers):
        assert_close(np64(gs.k_cache[l]), os_.k_cache[l], 1e-4, f"K cache {l} after sparse")
    # fp32 KL: rtol 1e-3 plus 1e-6 absolute.  The kernel combines three O(1) fp32 terms,
    # KL = t/s - (m - m') - log(s/s'), whose rounding (sums over V terms, hardware exp2 and log)
    # stays within about 16 ulps of (sum_v p_v |z_v - z'_v| + |m - m'| + 1), i.e. about 1e-6 here,
    # while the KL values of this step are ~2e-4.
    np.testing.assert_allclose(np64(gs.kl).reshape(-1)[info["rows"]], os_.kl.reshape(-1)[info["rows"]],
                               rtol=1e-3, atol=1e-6)


def _designed_conf(B, S, k, seed):
    """Confidences whose top-k per sequence are separated from the rest by a wide gap."""
    u = synth.uniform01(synth.seed_of(seed), (B, S)).numpy().astype(np.float64)
    conf = 0.3 * u
    for b in range(B):
        top = synth.permutation(synth.seed_of(seed, b), S)[:k].numpy()
        conf[b, top] = 0.6 + 0.4 * u[b, top]
    return conf.astype(np.float32)


@pytest.mark.parametrize("b_lay,vocab", [(0, 1000), (1, 1000), (3, 1000), (1, 32768)])
def test_bf16_early_skip_iteration(b_lay, vocab):
    # vocab 32768 with 48 active rows exercises the sliced vocabulary pass
    dims = workloads.shrink(workloads.LLADA, n_layers=3, d=256, n_heads=2, n_kv_heads=2, d_ff=512, vocab=vocab,
                            B=2, S=96, prompt=48)
    k = 24
    print(f"bf16 early-skip b={b_lay}", flush=True)
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=k, track_kl=True)
    ws = api.alloc_workspace(gm, dims.B, dims.S, k)
    os_ = new_state(om, tok.numpy(), track_kl=True)
    api.skip_step(gm, gs, api.step_cfg(b_lay, True, ws=ws))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=b_lay, full_step=True))
    torch.cuda.synchronize()
    _compare_state(gs, os_, np.arange(dims.B * dims.S), 2e-2, "full")
    # same designed confidences and the same newly unmasked tokens on both sides
    conf = _designed_conf(dims.B, dims.S, k, 77)
    gs.conf.copy_(torch.from_numpy(conf))
    os_.conf = conf.astype(np.float64)
    new_tok = tok.clone()
    new_tok[:, 50:53] = torch.tensor([5, 6, 7], dtype=torch.int32)
    gs.tokens.copy_(new_tok)
    os_.tokens = new_tok.numpy().astype(np.int64)
    k_before = [t.cpu().clone() for t in gs.k_cache]
    gsc, osc = _score_cfg_pair(0.5, VAR_L1N, SEL_TOPK, k)
    api.skip_step(gm, gs, api.step_cfg(b_lay, False, gsc, ws=ws))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=b_lay, full_step=False, score=osc))
    torch.cuda.synchronize()
    rows = info["rows"]
    got_rows = [b * dims.S + int(i) for b in range(dims.B) for i in gs.idx[b, :int(gs.n_active[b])].cpu()]
    assert got_rows == rows.tolist()
    _compare_state(gs, os_, rows, 2e-2, "sparse")
    _argmax_ok(gs, os_, rows, margin=0.05)
    skipped = np.setdiff1d(np.arange(dims.B * dims.S), rows)
    for l in range(dims.n_layers):
        kc = gs.k_cache[l].cpu().reshape(dims.B * dims.S, -1)
        assert_close(np64(kc)[rows], os_.k_cache[l].reshape(dims.B * dims.S, -1)[rows], 2e-2, f"K {l}")
        if l >= b_lay:   # skipped rows keep their cached K/V bit for bit
            assert torch.equal(kc[skipped], k_before[l].reshape(dims.B * dims.S, -1)[skipped])
    # the boundary state for the next iteration is the hidden state entering layer b
    assert_close(np64(gs.h_bnd_prev).reshape(dims.B * dims.S, -1), os_.h_bnd_prev.reshape(dims.B * dims.S, -1),
                 2e-2, "h_bnd")


@pytest.mark.parametrize("kl_state,vocab", [("f32", 1000), ("bf16", 1000), ("bf16", 16384)])
def test_bf16_gqa_surelock_iteration(kl_state, vocab):
    """SureLock iteration; the previous logits kept in fp32 or in bf16 (with V = 16384 the vocabulary
    pass splits every row into slices and merges them)."""
    print(f"surelock kl_state={kl_state} V={vocab}", flush=True)
    dims = workloads.shrink(workloads.DREAM, n_layers=2, d=256, n_heads=4, n_kv_heads=1, d_ff=384, vocab=vocab,
                            B=3, S=80, prompt=40)
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=dims.S, track_kl=True, kl_state=kl_state)
    ws = api.alloc_workspace(gm, dims.B, dims.S, dims.S)
    os_ = new_state(om, tok.numpy(), track_kl=True, kl_state_bf16=(kl_state == "bf16"))
    api.skip_step(gm, gs, api.step_cfg(0, True, ws=ws))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=True))
    # lock a seeded 40% of positions per sequence on both sides; change three tokens
    force = np.zeros((dims.B, dims.S), dtype=np.uint8)
    for b in range(dims.B):
        force[b, synth.permutation(synth.seed_of(88, b), dims.S)[:32].numpy()] = FORCE_EXCLUDED
    gs.force.copy_(torch.from_numpy(force))
    os_.force = force.copy()
    new_tok = tok.clone()
    new_tok[:, 45:48] = torch.tensor([1, 2, 3], dtype=torch.int32)
    gs.tokens.copy_(new_tok)
    os_.tokens = new_tok.numpy().astype(np.int64)
    kc_before = [t.cpu().clone() for t in gs.k_cache]
    zp_g, zp_o = np64(gs.logits_prev), os_.logits_prev.copy()   # the previous logits the KL compares with
    gsc, osc = _score_cfg_pair(0.0, VAR_L1N, SEL_UNLOCKED, dims.S)
    eps = 5e-3
    api.skip_step(gm, gs, api.step_cfg(0, False, gsc, lock_kl_eps=eps, lock_conf_min=-1.0, ws=ws))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=False, score=osc, lock_kl_eps=eps,
                                           lock_conf_min=-1.0))
    torch.cuda.synchronize()
    rows = info["rows"]
    assert len(rows) == dims.B * (dims.S - 32)
    got_rows = [b * dims.S + int(i) for b in range(dims.B) for i in gs.idx[b, :int(gs.n_active[b])].cpu()]
    assert got_rows == rows.tolist()
    _compare_state(gs, os_, rows, 2e-2, "surelock")
    # locked rows: cached K/V untouched at every layer
    locked = np.nonzero(force.reshape(-1) == FORCE_EXCLUDED)[0]
    for l in range(dims.n_layers):
        kc = gs.k_cache[l].cpu().reshape(dims.B * dims.S, -1)
        assert torch.equal(kc[locked], kc_before[l].reshape(dims.B * dims.S, -1)[locked])
    # KL: bf16 weights make the GPU's logits differ from the oracle's (within the logits tolerance
    # checked above); the KL may differ by what those logit differences explain to first order
    gkl = np64(gs.kl).reshape(-1)[rows]
    okl = os_.kl.reshape(-1)[rows]
    first, rest = kl_first_order(np64(gs.logits_prev)[rows], os_.logits_prev[rows], zp_g[rows], zp_o[rows],
                                  dims.mask_id)
    assert_within(gkl, okl + first, rest + 1e-3 * np.abs(okl), "surelock KL beyond its first-order change")
    # the lock rule: identical decisions wherever the oracle's KL is further from eps than the
    # GPU's KL can be
    gf = gs.force.cpu().numpy().reshape(-1)
    of = os_.force.reshape(-1)
    assert np.all(gf[locked] == FORCE_EXCLUDED)
    clear = np.abs(okl - eps) > np.abs(first) + rest + 1e-3 * np.abs(okl)
    assert np.mean(clear) > 0.9
    assert np.array_equal(gf[rows][clear], of[rows][clear])


def test_bf16_thresh_cap_forced_rows():
    """Cosine-gated partial update with forced (dilated-schedule) rows and excluded prompt rows."""
    dims = workloads.shrink(workloads.LLADA_LONG, n_layers=2, d=256, n_heads=2, n_kv_heads=2, d_ff=512,
                            vocab=1000, B=2, S=128, prompt=96)
    k = 12
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=k, track_kl=False)
    ws = api.alloc_workspace(gm, dims.B, dims.S, k)
    os_ = new_state(om, tok.numpy(), track_kl=False)
    api.skip_step(gm, gs, api.step_cfg(0, True, ws=ws))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=True))
    force = np.zeros((dims.B, dims.S), dtype=np.uint8)
    force[:, :dims.prompt] = FORCE_EXCLUDED
    force[:, [96, 104]] = 1
    gs.force.copy_(torch.from_numpy(force))
    os_.force = force.copy()
    new_tok = tok.clone()
    new_tok[:, [100, 112, 120]] = 9
    gs.tokens.copy_(new_tok)
    os_.tokens = new_tok.numpy().astype(np.int64)
    gsc, osc = _score_cfg_pair(0.0, VAR_COS, SEL_THRESH_CAP, k, tau=1e-4)
    api.skip_step(gm, gs, api.step_cfg(0, False, gsc, ws=ws))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=False, score=osc))
    torch.cuda.synchronize()
    rows = info["rows"]
    got_rows = [b * dims.S + int(i) for b in range(dims.B) for i in gs.idx[b, :int(gs.n_active[b])].cpu()]
    # the changed tokens and forced rows must be in; ties near tau are not expected at these sizes
    assert got_rows == rows.tolist()
    for b in range(dims.B):
        assert {b * dims.S + 96, b * dims.S + 104} <= set(got_rows)
        assert all(r % dims.S >= dims.prompt for r in got_rows)
    _compare_state(gs, os_, rows, 2e-2, "thresh")


def test_bf16_dilated_block_decode():
    """A block decoded by dilated rounds: each round recomputes a capped, cosine-gated set that always holds
    the round's planned positions, and unmasks exactly those positions."""
    dims = workloads.shrink(workloads.LLADA_LONG, n_layers=2, d=256, n_heads=2, n_kv_heads=2, d_ff=512,
                            vocab=1000, B=2, S=96, prompt=64)
    k, blk, a = 16, 16, 2
    lo, hi = dims.prompt, dims.prompt + blk
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=k, track_kl=True)
    ws = api.alloc_workspace(gm, dims.B, dims.S, k)
    os_ = new_state(om, tok.numpy(), track_kl=True)
    api.skip_step(gm, gs, api.step_cfg(0, True, ws=ws))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=True))
    gsc, osc = _score_cfg_pair(0.0, VAR_COS, SEL_THRESH_CAP, k, tau=1e-4)
    for rnd, plan in enumerate(dus_rounds(blk, a)):
        print(f"dilated round {rnd}: {plan}", flush=True)
        force = np.zeros((dims.B, dims.S), dtype=np.uint8)
        force[:, :dims.prompt] = FORCE_EXCLUDED
        force[:, [lo + p for p in plan]] = 1
        gs.force.copy_(torch.from_numpy(force))
        os_.force = force.copy()
        api.skip_step(gm, gs, api.step_cfg(0, False, gsc, unmask_n=1, block_lo=lo, block_hi=hi,
                                           unmask_mode=api.UNMASK_FORCED, ws=ws))
        os_, info = skip_step(om, os_, StepCfg(boundary_layer=0, full_step=False, score=osc, unmask_n=1,
                                               block_lo=lo, block_hi=hi, unmask_mode=UNMASK_FORCED))
        torch.cuda.synchronize()
        rows = info["rows"]
        got_rows = [b * dims.S + int(i) for b in range(dims.B) for i in gs.idx[b, :int(gs.n_active[b])].cpu()]
        assert got_rows == rows.tolist()
        for b in range(dims.B):
            assert {b * dims.S + lo + p for p in plan} <= set(got_rows)
        _compare_state(gs, os_, rows, 2e-2, f"round {rnd}")
        # the planned positions take the argmax: the oracle's token wherever its top-2 logit gap is clear of
        # rounding; in a near tie the GPU's pick is kept on both sides so later rounds see the same tokens
        gt = gs.tokens.cpu().numpy()
        planned = np.zeros((dims.B, dims.S), dtype=bool)
        planned[:, [lo + p for p in plan]] = True
        assert np.array_equal(gt[~planned], os_.tokens[~planned])
        assert np.array_equal(gt[planned], gs.argmax.cpu().numpy()[planned])
        for b, i in zip(*np.nonzero(planned)):
            z = os_.logits_prev[b * dims.S + i].copy()
            z[dims.mask_id] = -np.inf
            top2 = np.sort(z)[-2:]
            if top2[1] - top2[0] > 1e-2:
                assert gt[b, i] == os_.tokens[b, i], f"round {rnd} position {b},{i}"
            else:
                os_.tokens[b, i] = gt[b, i]
    assert not np.any(gs.tokens.cpu().numpy()[:, lo:hi] == dims.mask_id)


def test_all_rows_active_equals_full_step_on_gpu():
    """Property at any size: a sparse step with every row active reproduces a full step."""
    dims = workloads.shrink(workloads.LLADA, n_layers=2, d=256, n_heads=2, n_kv_heads=2, d_ff=512, vocab=1000,
                            B=1, S=64, prompt=32)
    gm, _ = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    outs = []
    for sparse in (False, True):
        gs = api.State(gm, tok.to(DEV), k_max=dims.S, track_kl=False)
        ws = api.alloc_workspace(gm, dims.B, dims.S, dims.S)
        api.skip_step(gm, gs, api.step_cfg(1, True, ws=ws))
        gs.tokens[:, 40] = 3
        if sparse:
            api.skip_step(gm, gs, api.step_cfg(1, False, api.score_cfg(k=dims.S), ws=ws))
        else:
            api.skip_step(gm, gs, api.step_cfg(1, True, ws=ws))
        torch.cuda.synchronize()
        outs.append((gs.h_fin.cpu(), gs.conf.cpu(), [t.cpu() for t in gs.k_cache]))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    for a, b in zip(outs[0][2], outs[1][2]):
        assert torch.equal(a, b)


def _tiered_conf(B, S, tiers, forced_top, seed):
    """Confidences in separated tiers: tiers = [n_1, n_2, ...] rows per sequence in bands
    [0.92, 1.0], [0.75, 0.83], [0.55, 0.63], ...; `forced_top` positions always in the top band;
    every other row in [0, 0.3]."""
    u = synth.uniform01(synth.seed_of(seed), (B, S)).numpy().astype(np.float64)
    conf = 0.3 * u
    for b in range(B):
        perm = [int(i) for i in synth.permutation(synth.seed_of(seed, b), S).numpy() if int(i) not in forced_top]
        order = list(forced_top) + perm
        start = 0
        for t, n in enumerate(tiers):
            lo = [0.92, 0.75, 0.55, 0.40][t]
            for i in order[start:start + n]:
                conf[b, i] = lo + 0.08 * u[b, i]
            start += n
    return conf.astype(np.float32)


def test_bf16_nested_boundaries():
    """Boundary at layer 1 (24 rows), nested boundaries at layers 2 (12 rows) and 3 (6 rows)."""
    dims = workloads.shrink(workloads.LLADA, n_layers=4, d=256, n_heads=2, n_kv_heads=2, d_ff=512, vocab=1000,
                            B=2, S=96, prompt=48)
    k, nested = 24, ((2, 12), (3, 6))
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=k, track_kl=True, n_nested=2)
    ws = api.alloc_workspace(gm, dims.B, dims.S, k)
    os_ = new_state(om, tok.numpy(), track_kl=True, n_nested=2)
    api.skip_step(gm, gs, api.step_cfg(1, True, ws=ws, nested=nested))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=1, full_step=True, nested=nested))
    torch.cuda.synchronize()
    BS = dims.B * dims.S
    for j in range(2):   # a full step fills the nested caches for every row
        assert_close(np64(gs.h_nested[j]).reshape(BS, -1), os_.h_nested[j].reshape(BS, -1), 2e-2, f"h_nested {j}")
    conf = _tiered_conf(dims.B, dims.S, [6, 6, 12], [50, 51, 52], 91)
    gs.conf.copy_(torch.from_numpy(conf))
    os_.conf = conf.astype(np.float64)
    new_tok = tok.clone()
    new_tok[:, 50:53] = torch.tensor([5, 6, 7], dtype=torch.int32)
    gs.tokens.copy_(new_tok)
    os_.tokens = new_tok.numpy().astype(np.int64)
    k_before = [t.cpu().clone() for t in gs.k_cache]
    hn_before = [t.cpu().clone() for t in gs.h_nested]
    hf_before = gs.h_fin.cpu().clone()
    gsc, osc = _score_cfg_pair(0.8, VAR_L1N, SEL_TOPK, k)
    api.skip_step(gm, gs, api.step_cfg(1, False, gsc, ws=ws, nested=nested))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=1, full_step=False, score=osc, nested=nested))
    torch.cuda.synchronize()
    # every selection is well separated, so both sides must take the same rows
    assert min(selection_gap(info["scores"][b], os_.force[b], k) for b in range(dims.B)) > 0.02
    for (rows_j, s_j), (_, kk) in zip(info["nested_scores"], nested):
        for b in range(dims.B):
            sb = np.sort(s_j[rows_j // dims.S == b])[::-1]
            assert sb[kk - 1] - sb[kk] > 0.02
    stage = [info["nested_scores"][0][0], info["nested_scores"][1][0], info["rows"]]  # rows entering 2, 3, final
    got_rows = [b * dims.S + int(i) for b in range(dims.B) for i in gs.idx[b, :int(gs.n_active[b])].cpu()]
    assert got_rows == info["rows"].tolist()
    final = info["rows"]
    _compare_state(gs, os_, final, 2e-2, "nested")
    others = np.setdiff1d(np.arange(BS), final)
    assert torch.equal(gs.h_fin.cpu().reshape(BS, -1)[others], hf_before.reshape(BS, -1)[others])
    for l in range(dims.n_layers):
        active = np.arange(BS) if l < 1 else (stage[0] if l < 2 else (stage[1] if l < 3 else final))
        kc = gs.k_cache[l].cpu().reshape(BS, -1)
        assert_close(np64(kc)[active], os_.k_cache[l].reshape(BS, -1)[active], 2e-2, f"K {l}")
        idle = np.setdiff1d(np.arange(BS), active)
        assert torch.equal(kc[idle], k_before[l].reshape(BS, -1)[idle]), f"layer {l} skipped rows"
    for j in range(2):   # caches refreshed exactly for the rows that reached the layer
        hn = gs.h_nested[j].cpu().reshape(BS, -1)
        reached = stage[j]
        assert_close(np64(hn)[reached], os_.h_nested[j].reshape(BS, -1)[reached], 2e-2, f"h_nested {j} rows")
        idle = np.setdiff1d(np.arange(BS), reached)
        assert torch.equal(hn[idle], hn_before[j].reshape(BS, -1)[idle])


@pytest.mark.parametrize("case", ["tiers_b1", "changed_b0", "value_tiers_b1", "value_changed_b0"])
def test_bf16_layer_cache(case):
    """Per-layer cache steps ([DC] section 3) against the oracle, prompt rows locked between full
    steps.  tiers_b1: layer 0 dense, layers 1-3 cached, alpha 0.8 with two separated confidence
    tiers (8 rows per sequence recomputed at every cached layer).  changed_b0: every layer cached,
    alpha 0 (cosine change only), k = the 3 positions whose tokens changed.  value_*: the same
    with the layers' V projections compared against the cached V instead of the hidden states."""
    dims = workloads.shrink(workloads.LLADA, n_layers=4, d=256, n_heads=2, n_kv_heads=2, d_ff=512, vocab=1000,
                            B=2, S=96, prompt=48)
    B, S, L = dims.B, dims.S, dims.n_layers
    BS = B * S
    feature = "value" if case.startswith("value_") else "hidden"
    case = case.replace("value_", "")
    b, k, alpha = (1, 8, 0.8) if case == "tiers_b1" else (0, 3, 0.0)
    print(f"layer cache {case}", flush=True)
    gm, om = _models(dims, std=0.05)
    tok = workloads.initial_tokens(dims)
    gs = api.State(gm, tok.to(DEV), k_max=k, track_kl=True, layer_cache=True)
    ws = api.alloc_workspace(gm, B, S, k)
    os_ = new_state(om, tok.numpy(), track_kl=True, layer_cache=True)
    api.skip_step(gm, gs, api.step_cfg(b, True, ws=ws, layer_cache=True))
    os_, _ = skip_step(om, os_, StepCfg(boundary_layer=b, full_step=True, layer_cache=True))
    torch.cuda.synchronize()
    for l in range(b, L):   # a full step fills both caches of every cached layer
        assert_close(np64(gs.x_in[l]).reshape(BS, -1), os_.x_in[l].reshape(BS, -1), 2e-2, f"x_in {l}")
        assert_close(np64(gs.x_out[l]).reshape(BS, -1), os_.x_out[l].reshape(BS, -1), 2e-2, f"x_out {l}")
    if case == "tiers_b1":
        # 8 response positions per sequence well above every other (the prompt rows are locked)
        u = synth.uniform01(synth.seed_of(93), (B, S)).numpy().astype(np.float64)
        conf = 0.3 * u
        for bb in range(B):
            for i in [50, 51, 52, 60 + bb, 66, 71, 77 + bb, 84]:
                conf[bb, i] = 0.75 + 0.25 * u[bb, i]
        conf = conf.astype(np.float32)
        gs.conf.copy_(torch.from_numpy(conf))
        os_.conf = conf.astype(np.float64)
    force = np.zeros((B, S), dtype=np.uint8)
    force[:, :dims.prompt] = 2                                  # long-interval prompt cache
    gs.force.copy_(torch.from_numpy(force))
    os_.force = force.copy()
    new_tok = tok.clone()
    new_tok[:, 50:53] = torch.tensor([5, 6, 7], dtype=torch.int32)
    gs.tokens.copy_(new_tok)
    os_.tokens = new_tok.numpy().astype(np.int64)
    kv_before = [(a.cpu().clone(), v.cpu().clone()) for a, v in zip(gs.k_cache, gs.v_cache)]
    xi_before = [t.cpu().clone() for t in gs.x_in]
    xo_before = [t.cpu().clone() for t in gs.x_out]
    hf_before = gs.h_fin.cpu().clone()
    gsc, osc = _score_cfg_pair(alpha, VAR_COS, SEL_TOPK, k)
    api.skip_step(gm, gs, api.step_cfg(b, False, gsc, ws=ws, layer_cache=feature))
    os_, info = skip_step(om, os_, StepCfg(boundary_layer=b, full_step=False, score=osc, layer_cache=True,
                                           cache_feature=feature))
    torch.cuda.synchronize()
    assert len(info["layer_rows"]) == L - b
    for s in info["layer_scores"]:        # every layer's selection is well separated
        assert min(selection_gap(s[bb], force[bb], k) for bb in range(B)) > 0.02
    got_rows = [bb * S + int(i) for bb in range(B) for i in gs.idx[bb, :int(gs.n_active[bb])].cpu()]
    assert got_rows == info["rows"].tolist()
    for l in range(L):
        rows_l = np.arange(BS) if l < b else info["layer_rows"][l - b]
        assert np.all(rows_l % S >= dims.prompt) or l < b
        idle = np.setdiff1d(np.arange(BS), rows_l)
        for t_g, t_o, t_b, nm in ((gs.k_cache[l], os_.k_cache[l], kv_before[l][0], "K"),
                                  (gs.v_cache[l], os_.v_cache[l], kv_before[l][1], "V")):
            g2 = t_g.cpu().reshape(BS, -1)
            assert_close(np64(g2)[rows_l], t_o.reshape(BS, -1)[rows_l], 2e-2, f"{nm} {l}")
            assert torch.equal(g2[idle], t_b.reshape(BS, -1)[idle]), f"{nm} layer {l} idle rows"
        if l >= b:
            for t_g, t_o, t_b, nm in ((gs.x_in[l], os_.x_in[l], xi_before[l], "x_in"),
                                      (gs.x_out[l], os_.x_out[l], xo_before[l], "x_out")):
                g2 = t_g.cpu().reshape(BS, -1)
                assert_close(np64(g2)[rows_l], t_o.reshape(BS, -1)[rows_l], 2e-2, f"{nm} {l}")
                assert torch.equal(g2[idle], t_b.reshape(BS, -1)[idle]), f"{nm} layer {l} idle rows"
    final = info["rows"]
    _compare_state(gs, os_, final, 2e-2, "layer cache")
    _argmax_ok(gs, os_, final, 0.05)
    others = np.setdiff1d(np.arange(BS), final)
    assert torch.equal(gs.h_fin.cpu().reshape(BS, -1)[others], hf_before.reshape(BS, -1)[others])
