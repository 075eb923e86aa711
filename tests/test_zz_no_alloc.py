"""dllm_layer_sparse_noalloc (the library's per-GPU scratch array instead of a workspace) against
dllm_layer_sparse (a caller workspace) on the same inputs (GPU).

Two calls in a row on one LLaDA-8B-shaped layer (d 4096, 32 heads, F 12288, S 512): 128 active
rows, then 40 live rows of a 64-row capacity, so the second call reuses scratch the first one
left behind.  The two entry points run the same kernels with the same launch plans, so the
residual stream and both caches must be bit-identical.
"""
import pytest
import torch

import synth
from synth import workloads
from tests.gpu_util import DEV
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def _inputs(dims, k_max, n_live, seed):
    B, S, d = dims.B, dims.S, dims.d
    x = synth.normal(synth.seed_of(seed, 1), (B * k_max, d), 1.0, torch.bfloat16)
    kc = synth.normal(synth.seed_of(seed, 2), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16)
    vc = synth.normal(synth.seed_of(seed, 3), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, torch.bfloat16)
    idx = torch.full((B, k_max), -1, dtype=torch.int32)
    idx[0, :n_live] = torch.sort(synth.permutation(synth.seed_of(seed, 4), S)[:n_live]).values.to(torch.int32)
    nact = torch.tensor([n_live], dtype=torch.int32)
    return [t.to(DEV) for t in (x, kc, vc, idx, nact)]


def test_noalloc_layer_matches_workspace_layer():
    dims = workloads.LLADA_LAYER
    print("no-alloc layer entry point vs workspace entry point", flush=True)
    lw = workloads.layer_weights(dims, 0, device=DEV)
    emb = torch.zeros((8, dims.d), dtype=torch.bfloat16, device=DEV)
    model = api.Model({"embed": emb, "final_norm": torch.ones(dims.d, dtype=torch.bfloat16, device=DEV),
                       "lm_head": emb, "layers": [lw]}, dims.n_heads, dims.n_kv_heads, 7)
    for k_max, n_live, seed in ((128, 128, 71), (64, 40, 72)):
        print(f"k_max {k_max}, live rows {n_live}", flush=True)
        x, kc, vc, idx, nact = _inputs(dims, k_max, n_live, seed)
        xr, kr, vr = x.clone(), kc.clone(), vc.clone()
        ws = api.alloc_workspace(model, dims.B, dims.S, k_max)
        api.layer_sparse(model, 0, xr, idx, nact, kr, vr, ws)
        xn, kn, vn = x.clone(), kc.clone(), vc.clone()
        api.layer_sparse_noalloc(model, 0, xn, idx, nact, kn, vn)
        torch.cuda.synchronize()
        assert torch.equal(xn[:n_live], xr[:n_live]), "residual stream of the live rows"
        assert torch.equal(kn, kr) and torch.equal(vn, vr), "K/V caches"
        assert not torch.equal(xn[:n_live], x[:n_live])   # the layer really ran


def test_noalloc_layer_rejects_shapes_beyond_the_scratch():
    """A dense 512-row call of the same layer needs about 75 MB of scratch: refused, nothing launched."""
    dims = workloads.LLADA_LAYER
    lw = workloads.layer_weights(dims, 0, device=DEV)
    emb = torch.zeros((8, dims.d), dtype=torch.bfloat16, device=DEV)
    model = api.Model({"embed": emb, "final_norm": torch.ones(dims.d, dtype=torch.bfloat16, device=DEV),
                       "lm_head": emb, "layers": [lw]}, dims.n_heads, dims.n_kv_heads, 7, pack=False)
    x, kc, vc, idx, nact = _inputs(dims, dims.S, dims.S, 73)
    before = x.clone()
    with pytest.raises(api.DllmError, match="workspace"):
        api.layer_sparse_noalloc(model, 0, x, idx, nact, kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(x, before)
