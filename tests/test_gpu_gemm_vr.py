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


def _shared_rows_bit_identical(dims, n_lo, n_hi, seed):
    """One layer on n_lo and on n_hi active rows of one sequence (the first n_lo rows and positions
    shared).  A first n_hi-row call leaves in the cache at the extra positions exactly what the
    n_hi-row layer writes there, so the two calls then attend over identical caches: the caches
    and the n_lo shared output rows must match bit for bit."""
    B, S, d = dims.B, dims.S, dims.d
    assert B == 1 and n_lo < n_hi <= S
    lw = workloads.layer_weights(dims, 0, device=DEV, seed_base=dims.cfg_id)
    emb = torch.zeros((8, d), dtype=torch.bfloat16, device=DEV)
    w = {"embed": emb, "final_norm": torch.ones(d, dtype=torch.bfloat16, device=DEV), "lm_head": emb, "layers": [lw]}
    model = api.Model(w, dims.n_heads, dims.n_kv_heads, 7)
    kv = (B, S, dims.n_kv_heads, dims.head_dim)
    kc0 = synth.normal(synth.seed_of(seed, 1), kv, 1.0, torch.bfloat16).to(DEV)
    vc0 = synth.normal(synth.seed_of(seed, 2), kv, 1.0, torch.bfloat16).to(DEV)
    x0 = synth.normal(synth.seed_of(seed, 3), (n_hi, d), 1.0, torch.bfloat16).to(DEV)
    pos = torch.sort(synth.permutation(synth.seed_of(seed, 4), S)[:n_hi]).values.to(torch.int32)

    def run(n, kc, vc):
        x = x0[:n].clone()
        idx = pos[:n].reshape(1, n).to(DEV)
        nact = torch.tensor([n], dtype=torch.int32, device=DEV)
        ws = api.alloc_workspace(model, B, S, n)
        api.layer_sparse(model, 0, x, idx, nact, kc, vc, ws)
        torch.cuda.synchronize()
        return x

    kc1, vc1 = kc0.clone(), vc0.clone()
    x_first = run(n_hi, kc1, vc1)
    kc_hi, vc_hi = kc1.clone(), vc1.clone()
    kc_lo, vc_lo = kc1.clone(), vc1.clone()
    x_hi = run(n_hi, kc_hi, vc_hi)
    x_lo = run(n_lo, kc_lo, vc_lo)
    # the fresh K/V a layer writes do not depend on what the cache held before
    assert torch.equal(x_hi, x_first)
    assert torch.equal(kc_hi, kc1) and torch.equal(vc_hi, vc1)
    assert torch.equal(kc_lo, kc_hi) and torch.equal(vc_lo, vc_hi)
    assert torch.equal(x_lo, x_hi[:n_lo])
    assert torch.all(torch.isfinite(x_lo.float()))
    # the layer did change the rows (the check is not vacuous)
    assert not torch.equal(x_lo, x0[:n_lo])


def test_register_staged_layer_bit_identical_to_direct_lds():
    """One LLaDA-8B-shaped layer (S 512, d 4096, SwiGLU 12288) on 255 and on 256 active rows.  From
    256 rows on, the 256 x 192 QKV (4 K splits) and gate/up + SwiGLU products and the 256 x 128 down
    product (4 K splits) run through registers; at 255 rows the same tiles and splits run
    direct-to-LDS.  O (128 x 128, 4 splits) and attention (32-query workgroups) are the same
    kernels at both counts and per row."""
    print("register-staged vs direct-to-LDS layer, 255 / 256 rows", flush=True)
    _shared_rows_bit_identical(workloads.LLADA_LAYER, 255, 256, 61)


def test_register_staged_wide_swiglu_bit_identical_to_direct_lds():
    """One Dream-7B-shaped layer (d 3584, GQA 28/4, SwiGLU 18944) on 2047 and on 2048 active rows of
    one sequence of 2048 positions: from 2048 rows on the gate/up + SwiGLU product runs on the
    register-staged 256 x 256 tiles, at 2047 rows on the 16-wave direct-to-LDS ones (same tiles,
    no K split); every other product and attention (128-query workgroups) take the same kernels
    and splits at both counts."""
    print("register-staged vs direct-to-LDS wide SwiGLU, 2047 / 2048 rows", flush=True)
    dims = workloads.shrink(workloads.DREAM, n_layers=1, B=1, S=2048, prompt=1024)
    _shared_rows_bit_identical(dims, 2047, 2048, 62)
