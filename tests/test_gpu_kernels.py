"""Parity of the score/select, gather/scatter and vocabulary kernels with the oracle (GPU)."""
import numpy as np
import pytest
import torch

import synth
from oracle.importance import FLT_MAX, importance_score
from oracle.selection import select_thresh_cap, select_topk
from oracle.vocab import conf_kl, kl_state_value
from tests.gpu_util import DEV, assert_close, np64, selection_gap
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def _scores_with_ties(seed, B, S):
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, -0.0, 0.25, 0.5, 0.5, 1.0, -1.0, np.inf, -np.inf, np.nan], dtype=np.float32)
    s = rng.uniform(-1, 1, (B, S)).astype(np.float32)
    s = np.round(s * 8) / 8  # many exact ties
    mask = rng.uniform(size=(B, S)) < 0.2
    s[mask] = vals[rng.integers(0, len(vals), int(mask.sum()))]
    force = rng.choice(np.array([0, 0, 0, 0, 0, 0, 1, 2], dtype=np.uint8), (B, S))
    return s.astype(np.float32), force


@pytest.mark.parametrize("B,S,k", [(1, 1, 1), (2, 7, 3), (3, 130, 0), (2, 1000, 125), (1, 1025, 1025),
                                   (4, 4096, 205), (2, 5000, 2500), (1, 512, 128)])
def test_topk_select_bit_exact(B, S, k):
    print(f"select B={B} S={S} k={k}", flush=True)
    s, force = _scores_with_ties(B * 1000 + S, B, S)
    conf = torch.from_numpy(s).to(DEV)
    h = torch.zeros((B, S, 8), dtype=torch.bfloat16, device=DEV)
    fo = torch.from_numpy(force).to(DEV)
    cfg = api.score_cfg(alpha=1.0, var=api.VAR_NONE, sel=api.SEL_TOPK, k=k)
    k_max = max(k, 1)
    score, idx, n_act = api.score_select(h, h, conf, cfg, force=fo, k_max=k_max)
    torch.cuda.synchronize()
    # alpha = 1 and no change term: the kernel's score equals the input (-0 becomes +0 in 1*c + 0*0)
    got = score.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(s))
    ok = ~np.isnan(s)
    assert np.array_equal(got[ok], s[ok])
    idx_c, n_c = idx.cpu().numpy(), n_act.cpu().numpy()
    for b in range(B):
        want = select_topk(s[b].astype(np.float64), force[b], k)
        assert n_c[b] == len(want)
        assert idx_c[b, :n_c[b]].tolist() == want.tolist()
        assert np.all(idx_c[b, n_c[b]:] == -1)


@pytest.mark.parametrize("B,S,k,tau", [(2, 300, 40, 0.3), (1, 4096, 205, 0.0), (3, 64, 64, 0.9)])
def test_thresh_cap_and_unlocked_select(B, S, k, tau):
    s, force = _scores_with_ties(S + 7, B, S)
    conf = torch.from_numpy(s).to(DEV)
    h = torch.zeros((B, S, 8), dtype=torch.bfloat16, device=DEV)
    fo = torch.from_numpy(force).to(DEV)
    cfg = api.score_cfg(alpha=1.0, var=api.VAR_NONE, sel=api.SEL_THRESH_CAP, k=k, tau=tau)
    _, idx, n_act = api.score_select(h, h, conf, cfg, force=fo, k_max=k)
    cfgu = api.score_cfg(alpha=1.0, var=api.VAR_NONE, sel=api.SEL_UNLOCKED)
    _, idx_u, n_u = api.score_select(h, h, conf, cfgu, force=fo, k_max=S)
    torch.cuda.synchronize()
    for b in range(B):
        want = select_thresh_cap(s[b].astype(np.float64), force[b], tau, k)
        assert idx[b, :int(n_act[b])].cpu().tolist() == want.tolist()
        want_u = select_topk(s[b].astype(np.float64), force[b], S)
        assert idx_u[b, :int(n_u[b])].cpu().tolist() == want_u.tolist()


def _hidden_pair(seed, B, S, w, dtype):
    hc = synth.normal(synth.seed_of(seed, 1), (B, S, w), 1.0, torch.float32)
    noise = synth.normal(synth.seed_of(seed, 2), (B, S, w), 1e-2, torch.float32)
    big = synth.normal(synth.seed_of(seed, 3), (B, S, w), 1.0, torch.float32)
    hp = hc + noise
    rows = torch.arange(S) % 37 == 5
    hp[:, rows] += big[:, rows]
    hp[:, 3] = hc[:, 3]                    # identical row
    if S > 9:
        hp[:, 9] = 0.0                      # zero-norm previous row
        hc[:, 8] = 0.0
    return hc.to(dtype), hp.to(dtype)


@pytest.mark.parametrize("dtype,w", [(torch.bfloat16, 4096), (torch.float32, 256), (torch.bfloat16, 3584)])
@pytest.mark.parametrize("var", [api.VAR_L1N, api.VAR_COS, api.VAR_L2REL, api.VAR_KL])
def test_score_parity(dtype, w, var):
    B, S, k = 2, 200, 25
    print(f"score dtype={dtype} w={w} var={var}", flush=True)
    hc, hp = _hidden_pair(w + var, B, S, w, dtype)
    conf = synth.uniform01(synth.seed_of(w, var, 9), (B, S))
    kl = synth.uniform01(synth.seed_of(w, var, 10), (B, S)) * 0.01
    cfg = api.score_cfg(alpha=0.5, conf_inverted=(var == api.VAR_COS), var=var, sel=api.SEL_TOPK, k=k)
    h_next = torch.empty_like(hc, device=DEV)
    score, idx, n_act = api.score_select(hc.to(DEV), hp.to(DEV), conf.to(DEV), cfg, kl_prev=kl.to(DEV),
                                         k_max=k, h_next=h_next)
    torch.cuda.synchronize()
    assert torch.equal(h_next.cpu(), hc)
    want = importance_score(np64(hc).reshape(B * S, w), np64(hp).reshape(B * S, w), np64(conf).reshape(-1),
                            np64(kl).reshape(-1), alpha=0.5, var=var, conf_inverted=(var == api.VAR_COS))
    got = np64(score).reshape(-1)
    # special rows are exact
    for b in range(B):
        assert got[b * S + 3] == pytest.approx(want[b * S + 3], abs=1e-7)
    finite = want < FLT_MAX / 2
    np.testing.assert_allclose(got[finite], want[finite], rtol=2e-5, atol=1e-6)
    assert np.array_equal(got[~finite], want[~finite])
    # selection: identical to the oracle's selection unless the oracle's boundary gap is a near tie
    for b in range(B):
        wsel = select_topk(want[b * S:(b + 1) * S], None, k)
        gap = selection_gap(want[b * S:(b + 1) * S], None, k)
        assert gap > 1e-5, f"designed inputs hit a near tie (gap {gap})"
        assert idx[b, :int(n_act[b])].cpu().tolist() == wsel.tolist()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_scatter_byte_exact(dtype):
    B, S, w, k_max = 3, 77, 264 if dtype == torch.float32 else 520, 20
    src = synth.normal(synth.seed_of(5), (B, S, w), 1.0, dtype).to(DEV)
    idx = torch.full((B, k_max), -1, dtype=torch.int32)
    n_act = torch.tensor([20, 0, 7], dtype=torch.int32)
    for b in range(B):
        n = int(n_act[b])
        idx[b, :n] = torch.sort(synth.permutation(synth.seed_of(6, b), S)[:n]).values.to(torch.int32)
    idx, n_act = idx.to(DEV), n_act.to(DEV)
    g = api.gather_rows(src, idx, n_act)
    dst = torch.zeros_like(src)
    api.scatter_rows(g, idx, n_act, dst)
    torch.cuda.synchronize()
    srcc, gc, dc = src.cpu(), g.cpu(), dst.cpu()
    for b in range(B):
        for j in range(int(n_act[b])):
            i = int(idx[b, j])
            assert torch.equal(gc[b * k_max + j], srcc[b, i])
        sel = idx[b, :int(n_act[b])].cpu().long()
        mask = torch.zeros(S, dtype=torch.bool)
        mask[sel] = True
        assert torch.equal(dc[b, mask], srcc[b, mask])
        assert torch.all(dc[b, ~mask] == 0)


@pytest.mark.parametrize("V,R,exclude", [(1024, 5, 1023), (126464, 6, 126463), (1001, 9, -1), (152064, 3, 7)])
def test_confidence_kl_parity(V, R, exclude):
    print(f"conf_kl V={V} R={R}", flush=True)
    B, S = 2, 8
    z = synth.normal(synth.seed_of(V, 1), (R, V), 2.0, torch.float32)
    zp_all = synth.normal(synth.seed_of(V, 2), (B * S, V), 2.0, torch.float32)
    row_pos = torch.tensor([(3 * r + 1) % (B * S) for r in range(R)], dtype=torch.int32)
    row_pos[1] = -1                                     # a dead row
    zp_all[row_pos[0]] = z[0]                           # identical logits -> KL exactly 0
    zp_all[row_pos[2]] = z[2] + 3.0                     # shifted logits -> KL ~ 0
    zd, zpd, rpd = z.to(DEV), zp_all.clone().to(DEV), row_pos.to(DEV)
    conf = torch.full((B * S,), -1.0, device=DEV)
    arg = torch.full((B * S,), -1, dtype=torch.int32, device=DEV)
    kl = torch.full((B * S,), -1.0, device=DEV)
    api.confidence_kl(zd, rpd, conf, arg, kl=kl, logits_prev=zpd, exclude_id=exclude, have_prev=True)
    torch.cuda.synchronize()
    live = [r for r in range(R) if row_pos[r] >= 0]
    pos = row_pos[live].long()
    wc, wa, wk = conf_kl(np64(z)[live], np64(zp_all)[pos.numpy()], exclude)
    assert_close(np64(conf)[pos], wc, 1e-5, "conf")
    assert np.array_equal(arg.cpu().numpy()[pos], wa)
    np.testing.assert_allclose(np64(kl)[pos], wk, rtol=1e-4, atol=2e-5)
    assert float(kl[row_pos[0]]) == 0.0
    # previous logits of live rows now hold this step's logits; dead row's slot untouched
    zpc = zpd.cpu()
    for r in live:
        assert torch.equal(zpc[row_pos[r]], z[r])
    untouched = sorted(set(range(B * S)) - set(pos.tolist()))
    assert torch.equal(zpc[untouched], zp_all[untouched])
    assert torch.all(conf.cpu()[untouched] == -1.0)
    # without a previous posterior KL is +inf
    api.confidence_kl(zd, rpd, conf, arg, kl=kl, logits_prev=None, exclude_id=exclude, have_prev=False)
    torch.cuda.synchronize()
    assert torch.all(torch.isinf(kl.cpu()[pos]))


@pytest.mark.parametrize("V,R,exclude", [(1024, 5, 1023), (126464, 6, 126463), (1001, 9, -1), (152064, 3, 7)])
def test_confidence_kl_bf16_state_parity(V, R, exclude):
    """Compact KL state: previous logits in bf16, KL between bf16(z) and the state; state written as bf16(z)."""
    print(f"conf_kl bf16 state V={V} R={R}", flush=True)
    B, S = 2, 8
    z = synth.normal(synth.seed_of(V, 3), (R, V), 2.0, torch.float32)
    zp_all = synth.normal(synth.seed_of(V, 4), (B * S, V), 2.0, torch.float32).to(torch.bfloat16)
    row_pos = torch.tensor([(5 * r + 2) % (B * S) for r in range(R)], dtype=torch.int32)
    row_pos[1] = -1                                     # a dead row
    zp_all[row_pos[0]] = z[0].to(torch.bfloat16)        # the state of identical logits -> KL exactly 0
    zp_all[row_pos[2]] = (z[2] + 3.0).to(torch.bfloat16)
    zd, zpd, rpd = z.to(DEV), zp_all.clone().to(DEV), row_pos.to(DEV)
    conf = torch.full((B * S,), -1.0, device=DEV)
    arg = torch.full((B * S,), -1, dtype=torch.int32, device=DEV)
    kl = torch.full((B * S,), -1.0, device=DEV)
    api.confidence_kl(zd, rpd, conf, arg, kl=kl, logits_prev=zpd, exclude_id=exclude, have_prev=True)
    torch.cuda.synchronize()
    live = [r for r in range(R) if row_pos[r] >= 0]
    pos = row_pos[live].long()
    wc, wa, wk = conf_kl(np64(z)[live], np64(zp_all)[pos.numpy()], exclude, prev_bf16=True)
    assert_close(np64(conf)[pos], wc, 1e-5, "conf")
    assert np.array_equal(arg.cpu().numpy()[pos], wa)
    np.testing.assert_allclose(np64(kl)[pos], wk, rtol=1e-4, atol=2e-5)
    assert float(kl[row_pos[0]]) == 0.0
    # the state now holds bf16(z) (RNE) bit for bit; the dead row's slot is untouched
    zpc = zpd.cpu()
    for r in live:
        want = torch.from_numpy(kl_state_value(np64(z[r:r + 1]), prev_bf16=True)[0]).to(torch.bfloat16)
        assert torch.equal(zpc[row_pos[r]].view(torch.int16), want.view(torch.int16))
    untouched = sorted(set(range(B * S)) - set(pos.tolist()))
    assert torch.equal(zpc[untouched].view(torch.int16), zp_all[untouched].view(torch.int16))
