"""Weights in MFMA fragment order (dllm_pack_weight) and the products that stream them (GPU).

The packed layout is checked element by element against its definition (an index map built
here with torch); layers whose four products use the packed copies are checked against the same
layers on the row-major copies (LLaDA-8B and Dream-7B shapes) and against the oracle (a
Dream-shaped layer here; the full-size LLaDA layer in test_gpu_fullsize.py).  The packed LM head
of a sparse step is checked against the row-major one here and against the oracle by the
full-size stack tests of test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import synth
from synth import workloads
from tests.gpu_util import DEV, assert_close, np64
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def _packed_reference(w, interleave_f):
    """Memory order stage kb, column block nb, step s, lane l, element e holds
    w[row(32 nb + l % 32)][16 (4 kb + s) + 8 (l // 32) + e]."""
    N, K = w.shape
    kb = torch.arange(K // 64).view(-1, 1, 1, 1, 1)
    nb = torch.arange(N // 32).view(1, -1, 1, 1, 1)
    s = torch.arange(4).view(1, 1, -1, 1, 1)
    lane = torch.arange(64).view(1, 1, 1, -1, 1)
    e = torch.arange(8).view(1, 1, 1, 1, -1)
    r = lane % 32
    if interleave_f:
        row = torch.where(r < 16, 16 * nb + r, interleave_f + 16 * nb + r - 16)
    else:
        row = 32 * nb + r
    col = 16 * (4 * kb + s) + 8 * (lane // 32) + e
    shape = (K // 64, N // 32, 4, 64, 8)
    return w[row.expand(shape), col.expand(shape)].reshape(N, K)


@pytest.mark.parametrize("N,K,f", [(64, 64, 0), (96, 192, 48), (256, 4096, 0), (384, 128, 192)])
def test_pack_layout_bit_exact(N, K, f):
    print(f"pack N={N} K={K} interleave={f}", flush=True)
    w = synth.normal(synth.seed_of(N, K, f), (N, K), 1.0, torch.bfloat16)
    got = api.pack_weight(w.to(DEV), interleave_f=f)
    torch.cuda.synchronize()
    want = _packed_reference(w, f)
    assert torch.equal(got.cpu().view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("bad", [dict(N=48, K=64, f=0), dict(N=64, K=32, f=0), dict(N=64, K=64, f=16),
                                 dict(N=96, K=64, f=40)])
def test_pack_rejects_bad_shapes(bad):
    w = torch.zeros((bad["N"], bad["K"]), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(api.DllmError):
        api.pack_weight(w, interleave_f=bad["f"])


def _packed_products(dims, rows):
    """The packed plans of the layer's three packed products over `rows` active rows."""
    nqkv = (dims.n_heads + 2 * dims.n_kv_heads) * dims.head_dim
    return {"qkv": api.packed_plan(rows, nqkv, dims.d),
            "gate_up": api.packed_plan(rows, 2 * dims.d_ff, dims.d, swiglu=True),
            "down": api.packed_plan(rows, dims.d, dims.d_ff)}


@pytest.mark.parametrize("shape,k", [("llada", 64), ("llada", 80), ("llada", 128), ("dream", 64), ("dream", 37)])
def test_packed_layer_matches_row_major(shape, k):
    """A layer on k active rows per sequence, the QKV, gate/up and down products on the packed
    weights (QKV and down into fp32 K-split partials, gate/up with the fused SwiGLU; O stays on its
    row-major tiles) against the row-major kernels on the
    same inputs: the LLaDA-8B layer (1 sequence of 512; 80 rows leave the last 32-row MFMA block
    partly clamped) and a Dream-7B GQA layer (2 sequences of 1024, ragged: 64 + 61 and 37 + 34 rows,
    the second case off every multiple of 16)."""
    if shape == "llada":
        dims, n_act = workloads.LLADA_LAYER, [k]
    else:
        dims, n_act = workloads.shrink(workloads.DREAM, n_layers=1, B=2), [k, k - 3]
    B, S, d = dims.B, dims.S, dims.d
    plans = _packed_products(dims, B * k)
    print(f"packed vs row-major layer {shape} k={k} plans={plans}", flush=True)
    assert all(p is not None for p in plans.values())
    lw = workloads.layer_weights(dims, 0, device=DEV, seed_base=dims.cfg_id)
    emb = torch.zeros((8, d), dtype=torch.bfloat16, device=DEV)
    w = {"embed": emb, "final_norm": torch.ones(d, dtype=torch.bfloat16, device=DEV), "lm_head": emb, "layers": [lw]}
    m_pk = api.Model(w, dims.n_heads, dims.n_kv_heads, 7, pack=True)
    m_rm = api.Model(w, dims.n_heads, dims.n_kv_heads, 7, pack=False)
    names = ("w_gate_up_packed", "w_down_packed", "w_qkv_packed")
    assert all(getattr(m_pk._lw[0], n) for n in names)
    assert not any(getattr(m_rm._lw[0], n) for n in names)
    kc0 = synth.normal(synth.seed_of(5, 1), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).to(DEV)
    vc0 = synth.normal(synth.seed_of(5, 2), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).to(DEV)
    x0 = synth.normal(synth.seed_of(5, 3), (B * k, d), 1.0, torch.bfloat16).to(DEV)
    idx = torch.full((B, k), -1, dtype=torch.int32)
    for b in range(B):
        idx[b, :n_act[b]] = torch.sort(synth.permutation(synth.seed_of(5, 4, b), S)[:n_act[b]]).values.to(torch.int32)
    idx = idx.to(DEV)
    nact = torch.tensor(n_act, dtype=torch.int32, device=DEV)
    outs = []
    for m in (m_pk, m_rm):
        x, kc, vc = x0.clone(), kc0.clone(), vc0.clone()
        ws = api.alloc_workspace(m, B, S, k)
        api.layer_sparse(m, 0, x, idx, nact, kc, vc, ws)
        torch.cuda.synchronize()
        outs.append((x, kc, vc))
    (xp, kp, vp), (xr, kr, vr) = outs
    # the two QKV paths sum the reduction in different orders (other K splits), so a stored bf16
    # K/V element may round one ulp (2^-8 of itself) the other way; untouched rows stay identical
    for b in range(B):
        written = torch.zeros(S, dtype=torch.bool, device=DEV)
        written[idx[b, :n_act[b]].long()] = True
        for a, c in ((kp, kr), (vp, vr)):
            assert_close(np64(a[b][written]), np64(c[b][written]), 5e-3, "fresh K/V, packed vs row-major")
            assert torch.equal(a[b][~written], c[b][~written])
    # two bf16 evaluation orders of the same layer: the flipped Q/K/V roundings move the attention
    # weights and its output, which carry into the residual stream as they do against the oracle
    # (about 5e-3 of the largest element for this layer), so the bf16 bar applies
    live = torch.cat([torch.arange(b * k, b * k + n_act[b]) for b in range(B)]).to(DEV)
    assert_close(np64(xp[live]), np64(xr[live]), 2e-2, "layer output, packed vs row-major")
    assert torch.all(torch.isfinite(xp[live].float()))


def test_packed_dream_layer_128_rows_oracle():
    """A Dream-7B-shaped GQA layer (d 3584, 28 / 4 heads, SwiGLU 18944) over 2 sequences of 1024
    with 64 and 61 active rows: the three packed products on the packed path (their plans differ from the
    LLaDA ones: QKV 3 waves x 4 K splits, gate/up 2-wave workgroups), checked against the oracle on the
    K/V of every active row and the outputs of sampled rows."""
    from tests.test_gpu_fullsize import _sampled_layer_case
    dims = workloads.shrink(workloads.DREAM, n_layers=1, B=2)
    plans = _packed_products(dims, 2 * 64)
    print(f"dream layer 128 rows packed vs oracle plans={plans}", flush=True)
    assert all(p is not None for p in plans.values())
    _sampled_layer_case(dims, [64, 61], n_sample=8, seed=66)


@pytest.mark.parametrize("shape", ["llada", "dream"])
def test_packed_lm_head_matches_row_major(shape):
    """The LM head over the computed rows of a sparse step (at most 128) streams the packed copy
    (128-column tiles, one K split); over the 512 or 2048 rows of a full step it keeps the
    row-major tiles.  Two-layer models at the LLaDA-8B (V 126464, d 4096; 1 sequence, k = 128) and
    Dream-7B (V 152064, d 3584; 2 sequences, k = 64) shapes, a full step then a sparse step with
    the boundary after layer 1, with and without the packed LM head: both kernels sum every logit
    in one fp32 MFMA chain over K in the same order, so confidence, argmax, KL and the unmasked
    tokens agree bit for bit."""
    if shape == "llada":
        dims, k = workloads.shrink(workloads.LLADA, n_layers=2), 128
    else:
        dims, k = workloads.shrink(workloads.DREAM, n_layers=2, B=2), 64
    B, S = dims.B, dims.S
    plan = api.packed_plan(B * k, dims.vocab, dims.d)
    print(f"packed lm head {shape} rows={B * k} plan={plan}", flush=True)
    assert plan is not None
    w = workloads.model_weights(dims, device=DEV)
    m_pk = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    assert m_pk.lm_head_packed is not None
    m_rm = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    m_rm.lm_head_packed = None
    m_rm.c.lm_head_packed = None
    tok = workloads.initial_tokens(dims, device=DEV)
    lo, hi = dims.prompt, dims.prompt + 32
    outs = []
    for m in (m_pk, m_rm):
        st = api.State(m, tok.clone(), k_max=k, track_kl=True)
        ws = api.alloc_workspace(m, B, S, k)
        api.skip_step(m, st, api.step_cfg(1, True, unmask_n=4, block_lo=lo, block_hi=hi, ws=ws))
        sc = api.score_cfg(alpha=0.5, var=api.VAR_L1N, sel=api.SEL_TOPK, k=k)
        api.skip_step(m, st, api.step_cfg(1, False, sc, unmask_n=4, block_lo=lo, block_hi=hi, ws=ws))
        torch.cuda.synchronize()
        outs.append(st)
    a, b = outs
    assert torch.equal(a.n_active, b.n_active) and torch.equal(a.idx, b.idx)
    assert torch.equal(a.conf, b.conf) and torch.equal(a.argmax, b.argmax)
    assert torch.equal(a.kl, b.kl)
    assert torch.equal(a.tokens, b.tokens)
