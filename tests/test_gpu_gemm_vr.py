"""The register-staged GEMM (k_gemm_vr) against the direct-to-LDS one through the C ABI (GPU).

Both kernels reduce every output element over the same K splits in the same k order, so a layer
whose products change kernel between two row counts must give bit-identical rows for the rows the
two calls share."""
import pytest
import torch

import synth
from synth import workloads
from tests.gpu_util import DEV
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def test_register_staged_layer_bit_identical_to_direct_lds():
    """One LLaDA-8B-shaped layer (S 512, d 4096, SwiGLU 12288) on 255 and on 256 active rows of one
    sequence.  From 256 rows on, the 256 x 192 QKV (4 K splits) and gate/up + SwiGLU products and the
    256 x 128 down product (4 K splits) run through registers; at 255 rows the same tiles and splits
    run direct-to-LDS.  O (128 x 128, 4 splits) and attention (32-query workgroups) are the same
    kernels at both counts and per row.  A first 256-row call leaves in the cache at the 256th
    position exactly what the 256-row layer writes there, so the two calls then attend over
    identical caches: the caches and the 255 shared output rows must match bit for bit."""
    dims = workloads.LLADA_LAYER
    B, S, d = dims.B, dims.S, dims.d
    assert B == 1
    lw = workloads.layer_weights(dims, 0, device=DEV, seed_base=dims.cfg_id)
    emb = torch.zeros((8, d), dtype=torch.bfloat16, device=DEV)
    w = {"embed": emb, "final_norm": torch.ones(d, dtype=torch.bfloat16, device=DEV), "lm_head": emb, "layers": [lw]}
    model = api.Model(w, dims.n_heads, dims.n_kv_heads, 7)
    kv = (B, S, dims.n_kv_heads, dims.head_dim)
    kc0 = synth.normal(synth.seed_of(61, 1), kv, 1.0, torch.bfloat16).to(DEV)
    vc0 = synth.normal(synth.seed_of(61, 2), kv, 1.0, torch.bfloat16).to(DEV)
    x0 = synth.normal(synth.seed_of(61, 3), (256, d), 1.0, torch.bfloat16).to(DEV)
    pos = torch.sort(synth.permutation(synth.seed_of(61, 4), S)[:256]).values.to(torch.int32)
    print("register-staged vs direct-to-LDS layer, 255 / 256 rows", flush=True)

    def run(n, kc, vc):
        x = x0[:n].clone()
        idx = pos[:n].reshape(1, n).to(DEV)
        nact = torch.tensor([n], dtype=torch.int32, device=DEV)
        ws = api.alloc_workspace(model, B, S, n)
        api.layer_sparse(model, 0, x, idx, nact, kc, vc, ws)
        torch.cuda.synchronize()
        return x

    kc1, vc1 = kc0.clone(), vc0.clone()
    x_first = run(256, kc1, vc1)
    kc256, vc256 = kc1.clone(), vc1.clone()
    kc255, vc255 = kc1.clone(), vc1.clone()
    x256 = run(256, kc256, vc256)
    x255 = run(255, kc255, vc255)
    # the fresh K/V a layer writes do not depend on what the cache held before
    assert torch.equal(x256, x_first)
    assert torch.equal(kc256, kc1) and torch.equal(vc256, vc1)
    assert torch.equal(kc255, kc256) and torch.equal(vc255, vc256)
    assert torch.equal(x255, x256[:255])
    assert torch.all(torch.isfinite(x255.float()))
    # the layer did change the rows (the check is not vacuous)
    assert not torch.equal(x255, x0[:255])
