"""Weights in MFMA fragment order (dllm_pack_weight) and the products that stream them (GPU).

The packed layout is checked element by element against its definition (an index map built
here with torch); the layer that uses the packed gate/up and down copies is checked against the
same layer on the row-major copies, and the full-size LLaDA layer test (test_gpu_fullsize.py)
checks it against the oracle.
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


@pytest.mark.parametrize("k", [64, 128])
def test_packed_layer_matches_row_major(k):
    """The LLaDA-8B-shaped layer on k active rows: packed QKV (2 K splits), packed gate/up (fused
    SwiGLU) and packed down (8 K splits) against the row-major kernels on the same inputs."""
    dims = workloads.LLADA_LAYER
    B, S, d = dims.B, dims.S, dims.d
    print(f"packed vs row-major layer k={k}", flush=True)
    lw = workloads.layer_weights(dims, 0, device=DEV, seed_base=dims.cfg_id)
    emb = torch.zeros((8, d), dtype=torch.bfloat16, device=DEV)
    w = {"embed": emb, "final_norm": torch.ones(d, dtype=torch.bfloat16, device=DEV), "lm_head": emb, "layers": [lw]}
    m_pk = api.Model(w, dims.n_heads, dims.n_kv_heads, 7, pack=True)
    m_rm = api.Model(w, dims.n_heads, dims.n_kv_heads, 7, pack=False)
    assert m_pk._lw[0].w_gate_up_packed and m_pk._lw[0].w_down_packed and m_pk._lw[0].w_qkv_packed
    assert not m_rm._lw[0].w_gate_up_packed and not m_rm._lw[0].w_down_packed and not m_rm._lw[0].w_qkv_packed
    kc0 = synth.normal(synth.seed_of(5, 1), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).to(DEV)
    vc0 = synth.normal(synth.seed_of(5, 2), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16).to(DEV)
    x0 = synth.normal(synth.seed_of(5, 3), (B * k, d), 1.0, torch.bfloat16).to(DEV)
    idx = torch.sort(synth.permutation(synth.seed_of(5, 4), S)[:k]).values.to(torch.int32).view(1, k).to(DEV)
    nact = torch.full((B,), k, dtype=torch.int32, device=DEV)
    outs = []
    for m in (m_pk, m_rm):
        x, kc, vc = x0.clone(), kc0.clone(), vc0.clone()
        ws = api.alloc_workspace(m, B, S, k)
        api.layer_sparse(m, 0, x, idx, nact, kc, vc, ws)
        torch.cuda.synchronize()
        outs.append((x, kc, vc))
    (xp, kp, vp), (xr, kr, vr) = outs
    # the two QKV paths sum the reduction in different orders (2 vs 4 K splits), so a stored bf16
    # K/V element may round one ulp (2^-8 of itself) the other way; untouched rows stay identical
    written = torch.zeros(S, dtype=torch.bool)
    written[idx[0].cpu().long()] = True
    for a, b in ((kp, kr), (vp, vr)):
        assert_close(np64(a[0][written.to(DEV)]), np64(b[0][written.to(DEV)]), 5e-3, "fresh K/V, packed vs row-major")
        assert torch.equal(a[0][~written.to(DEV)], b[0][~written.to(DEV)])
    # two bf16 evaluation orders of the same layer: the flipped Q/K/V roundings move the attention
    # weights and its output, which carry into the residual stream as they do against the oracle
    # (about 5e-3 of the largest element for this layer), so the bf16 bar applies
    assert_close(np64(xp), np64(xr), 2e-2, "layer output, packed vs row-major")
    assert torch.all(torch.isfinite(xp.float()))
