"""dllm_layer_sparse (one layer on the active rows) against the oracle's partial update (GPU)."""
import numpy as np
import pytest
import torch

import synth
from oracle.numerics import store_fn
from oracle.transformer import layer_rows
from synth import workloads
from tests.gpu_util import DEV, assert_close, np64
from tests.helpers import oracle_weights
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu

CASES = {
    # name: (dims, weight std, n_active per sequence, k_max)
    "bf16_mha_ragged": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=2, n_kv_heads=2, d_ff=512,
                                         vocab=1000, B=2, S=100, prompt=50), 0.1, [37, 20], 37),
    "bf16_gqa7": (workloads.shrink(workloads.DREAM, n_layers=1, d=256, n_heads=7, n_kv_heads=1, d_ff=384,
                                   vocab=1000, B=3, S=130, prompt=64), 0.1, [50, 1, 0], 50),
    "bf16_full_rows": (workloads.shrink(workloads.LLADA, n_layers=1, d=512, n_heads=4, n_kv_heads=4, d_ff=1024,
                                        vocab=1000, B=1, S=192, prompt=96), 0.05, [192], 192),
    "f32_tiny": (workloads.shrink(workloads.TINY, n_layers=1, B=2, S=70), 0.1, [17, 30], 30),
    # 65 KV heads of one 128-query block over 34 key tiles (ragged): too few workgroups for the
    # chip, so each key range is split across 2 workgroups (split-KV + merge)
    "bf16_split_kv": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=65, n_kv_heads=65, d_ff=384,
                                       vocab=1000, B=1, S=2120, prompt=1024), 0.1, [40], 40),
    # 4 x 17 query blocks of 128: enough workgroups for the 128-query kernel without a split
    "bf16_q128": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=17, n_kv_heads=17, d_ff=384,
                                   vocab=1000, B=4, S=100, prompt=50), 0.1, [37, 20, 1, 9], 37),
    # 600 rows (two sequences of k_max 300, the second with 7 live rows): the many-row plans
    # (256 x 192 interleaved SwiGLU, 256 x 128 split-K down, 128 x 128 QKV and O) over a
    # ragged last tile and whole dead tiles; attention in 32-query workgroups over 300 slots
    "bf16_ragged_256_tiles": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=2, n_kv_heads=2, d_ff=768,
                                               vocab=1000, B=2, S=400, prompt=200), 0.05, [300, 7], 300),
    # F = 640 (a multiple of 128, not of 96) over 560 rows: interleaved 128 x 256 SwiGLU tiles
    "bf16_ffn640_many_rows": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=2, n_kv_heads=2, d_ff=640,
                                               vocab=1000, B=2, S=300, prompt=150), 0.05, [280, 151], 280),
    # F = 320 (a multiple of neither 96 nor 128) over 560 rows: the many-row SwiGLU fallback
    # (128 x 128 tiles, gate and up in the two halves of each wave's columns, two k-groups)
    "bf16_ffn320_many_rows": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=2, n_kv_heads=2, d_ff=320,
                                               vocab=1000, B=2, S=300, prompt=150), 0.05, [280, 151], 280),
    # two key tiles, one partial, over four waves: two waves of each workgroup have no keys
    "bf16_one_tile": (workloads.shrink(workloads.LLADA, n_layers=1, d=256, n_heads=2, n_kv_heads=2, d_ff=512,
                                       vocab=1000, B=2, S=40, prompt=20), 0.1, [13, 40], 40),
}


def _case(name):
    dims, std, nact, k_max = CASES[name]
    dt = workloads.torch_dtype(dims)
    w = workloads.model_weights(dims, std=std)
    B, S, d = dims.B, dims.S, dims.d
    x_act = synth.normal(synth.seed_of(31, dims.cfg_id), (B * k_max, d), 1.0, dt)
    idx = torch.full((B, k_max), -1, dtype=torch.int32)
    for b in range(B):
        idx[b, :nact[b]] = torch.sort(synth.permutation(synth.seed_of(32, b), S)[:nact[b]]).values.to(torch.int32)
    kc = synth.normal(synth.seed_of(33), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, dt)
    vc = synth.normal(synth.seed_of(34), (B, S, dims.n_kv_heads, dims.head_dim), 1.0, dt)
    return dims, w, x_act, idx, torch.tensor(nact, dtype=torch.int32), kc, vc, k_max


@pytest.mark.parametrize("name", list(CASES))
def test_layer_sparse_parity(name):
    print(f"layer case {name}", flush=True)
    dims, w, x_act, idx, nact, kc, vc, k_max = _case(name)
    B, S, d = dims.B, dims.S, dims.d
    live = [b * k_max + j for b in range(B) for j in range(int(nact[b]))]
    dead = sorted(set(range(B * k_max)) - set(live))
    x_in = x_act.clone()
    x_in[dead] = float("nan")            # dead rows must not leak into live ones

    model = api.Model({k: (v.to(DEV) if torch.is_tensor(v) else [{a: t.to(DEV) for a, t in lw.items()} for lw in v])
                       for k, v in w.items()}, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    xg, kcg, vcg = x_in.to(DEV), kc.clone().to(DEV), vc.clone().to(DEV)
    ws = api.alloc_workspace(model, B, S, k_max)
    api.layer_sparse(model, 0, xg, idx.to(DEV), nact.to(DEV), kcg, vcg, ws)
    torch.cuda.synchronize()

    mode = "exact" if dims.dtype == "f32" else "bf16"
    tol = 1e-4 if mode == "exact" else 2e-2
    ow = oracle_weights(w)
    pos = np.array([int(idx[r // k_max, r % k_max]) for r in live])
    bat = np.array([r // k_max for r in live])
    kco, vco = np64(kc), np64(vc)
    xo = layer_rows(ow["layers"][0], np64(x_act)[live], pos, bat, kco, vco, n_heads=dims.n_heads,
                    n_kv_heads=dims.n_kv_heads, rope_base=1e4, eps=1e-5, store=store_fn(mode))
    xgc = np64(xg)
    assert np.all(np.isfinite(xgc[live]))
    assert_close(xgc[live], xo, tol, f"{name}: residual stream")
    # written cache rows match; every other cache row is byte-identical to its input
    written = np.zeros((B, S), dtype=bool)
    written[bat, pos] = True
    for got, want, before in ((kcg, kco, kc), (vcg, vco, vc)):
        g = got.cpu()
        assert_close(np64(g)[written], want[written], tol, f"{name}: cache rows")
        assert torch.equal(g[torch.from_numpy(~written)], before[torch.from_numpy(~written)])
