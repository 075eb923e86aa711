"""Attention of the active queries over the whole K/V cache, isolated through dllm_layer_sparse (GPU).

The layer is set up so that its output is the attention output: d = Hq * D, the output
projection is the identity and the SwiGLU weights are zero, so x_out = x_in + O (x_in is kept
small; RMSNorm makes Q, K, V independent of its scale).  The cached keys are designed so that,
for every (query, head), a key in a late tile of every key range a wave, a key group or a
split-KV workgroup walks scores far above every key of that range's first tile: the running
maximum of the online softmax then jumps by more than the kernels' lazy-rescale threshold
(2^8 in the exp2 domain, 5.55 nats) inside every range, so the accumulator rescale runs.

Cases cover the three bf16 attention paths: 32-query workgroups (GQA 8/2), 128-query
workgroups without a key split, and split-KV with the merge kernel.  Every element of the output
is checked against the oracle's attention (SureLock technical summary 2.1 items 3-4: active
queries over all cached keys) within a bound derived from the bf16 roundings the two sides do
not share.
"""
import numpy as np
import pytest
import torch

import synth
from oracle.numerics import store_fn
from oracle.transformer import attention_rows, layer_rows, rmsnorm, rope
from tests.gpu_util import DEV, assert_close, assert_within, np64
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu
STORE = store_fn("bf16")
D = 128
WINDOW, HOT0 = 256, 128           # keys p with p % 256 >= 128 are "hot" slots, the rest cold
TARGET = 12.0                     # designed score (nats) of a query's own hot key in every window

CASES = {
    # name: (B, S, Hq, Hkv, n_active per sequence, k_max); the launch path follows from the shape
    "q32_gqa4": (1, 1024, 8, 2, [32], 32),
    "q128_unsplit": (4, 768, 17, 17, [37, 20, 1, 9], 37),
    "split_kv": (2, 2048, 33, 33, [40, 23], 40),
}


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("name", list(CASES))
def test_attention_isolated(name):
    B, S, Hq, Hkv, nact, k_max = CASES[name]
    print(f"attention case {name}", flush=True)
    g = Hq // Hkv
    d = Hq * D
    seed = 600 + list(CASES).index(name)
    assert k_max * g <= WINDOW - HOT0, "one hot slot per (query, head) in every window"
    # weights: Q/K/V projections N(0, 1/d) (unit-variance Q, K, V from unit-rms inputs),
    # identity output projection, zero SwiGLU
    wq = synth.normal(synth.seed_of(seed, 1), (Hq * D, d), d ** -0.5, torch.bfloat16)
    wk = synth.normal(synth.seed_of(seed, 2), (Hkv * D, d), d ** -0.5, torch.bfloat16)
    wv = synth.normal(synth.seed_of(seed, 3), (Hkv * D, d), d ** -0.5, torch.bfloat16)
    lw = {"attn_norm": torch.ones(d, dtype=torch.bfloat16), "wq": wq, "wk": wk, "wv": wv,
          "wo": torch.eye(d, dtype=torch.bfloat16), "ffn_norm": torch.ones(d, dtype=torch.bfloat16),
          "wg": torch.zeros((64, d), dtype=torch.bfloat16), "wu": torch.zeros((64, d), dtype=torch.bfloat16),
          "wd": torch.zeros((d, 64), dtype=torch.bfloat16)}
    lwo = {k: v.double().numpy() for k, v in lw.items()}

    # active positions: cold slots only (their fresh K/V overwrite the cache rows)
    idx = torch.full((B, k_max), -1, dtype=torch.int32)
    pos_l, bat_l = [], []
    for b in range(B):
        cold = np.array([p for p in synth.permutation(synth.seed_of(seed, 4, b), S).numpy() if p % WINDOW < HOT0])
        p_b = np.sort(cold[:nact[b]])
        idx[b, :nact[b]] = torch.from_numpy(p_b.astype(np.int32))
        pos_l.append(p_b)
        bat_l.append(np.full(nact[b], b))
    pos, bat = np.concatenate(pos_l), np.concatenate(bat_l)
    live = np.concatenate([b * k_max + np.arange(nact[b]) for b in range(B)])
    x_act = synth.normal(synth.seed_of(seed, 5), (B * k_max, d), 0.01, torch.bfloat16)
    kc = synth.normal(synth.seed_of(seed, 6), (B, S, Hkv, D), 1.0, torch.bfloat16).double().numpy()
    vc = synth.normal(synth.seed_of(seed, 7), (B, S, Hkv, D), 1.0, torch.bfloat16).double().numpy()

    # the active queries after RoPE, as both sides store them (bf16)
    x64 = x_act.double().numpy()[live]
    n = STORE(rmsnorm(x64, lwo["attn_norm"], 1e-5))
    q = STORE(rope((n @ lwo["wq"].T).reshape(-1, Hq, D), pos, 1e4))
    # hot keys: in every window, slot HOT0 + j g + hh of KV head hk points along query j's head
    # hk g + hh, scaled so that their score is TARGET nats
    for r in range(len(live)):
        b, j = bat[r], int(live[r] - bat[r] * k_max)
        for h in range(Hq):
            hk, hh = h // g, h % g
            qv = q[r, h]
            kv = qv * (TARGET * np.sqrt(D) / float(qv @ qv))
            for w0 in range(0, S, WINDOW):
                p = w0 + HOT0 + j * g + hh
                if p < S:
                    kc[b, p, hk] = kv
    kc = STORE(kc)

    # GPU: the layer on the active rows
    model = api.Model({"embed": torch.zeros((8, d), dtype=torch.bfloat16, device=DEV),
                       "final_norm": torch.ones(d, dtype=torch.bfloat16, device=DEV),
                       "lm_head": torch.zeros((8, d), dtype=torch.bfloat16, device=DEV),
                       "layers": [{k: v.to(DEV) for k, v in lw.items()}]}, Hq, Hkv, 7)
    xg = x_act.to(DEV)
    kcg, vcg = _bf16(kc).to(DEV), _bf16(vc).to(DEV)
    ws = api.alloc_workspace(model, B, S, k_max)
    api.layer_sparse(model, 0, xg, idx.to(DEV), torch.tensor(nact, dtype=torch.int32).to(DEV), kcg, vcg, ws)
    torch.cuda.synchronize()

    # oracle: the same layer (its attention over the cache with the fresh rows written)
    kco, vco = kc.copy(), vc.copy()
    want = layer_rows(lwo, x64, pos, bat, kco, vco, n_heads=Hq, n_kv_heads=Hkv, rope_base=1e4, eps=1e-5,
                      store=STORE)
    # the design holds: in every window, each (query, head)'s own hot key scores at least 6 nats
    # above every key of the window's first 64 (the first tile of any key range that starts
    # there: a q32 wave, either key group of a 128-query tile, a split-KV workgroup)
    for r in range(len(live)):
        b = bat[r]
        for h in range(Hq):
            s = kco[b, :, h // g] @ q[r, h] / np.sqrt(D)
            for w0 in range(0, S, WINDOW):
                first = np.max(s[w0:min(w0 + 64, S)])
                hot = np.max(s[w0 + HOT0:min(w0 + WINDOW, S)]) if w0 + HOT0 < S else -np.inf
                assert hot - first >= 6.0, f"design: window {w0}, row {r}, head {h}: {hot - first:.2f} nats"
    got = np64(xg)[live]
    assert np.all(np.isfinite(got))
    assert_close(got, want, 2e-2, f"{name}: attention output")
    # element-wise bound: both sides round the softmax weights to bf16 (against power-of-two
    # references), but a weight whose fp32 exponent argument lands next to a rounding boundary
    # may round the other way (at most 2^-8 of that weight, so |dO| <= 2^-8 sum_j p_j |V_j|), and
    # the stored O and x = x_in + O may each round one ulp (2^-8) the other way; twice that, plus
    # the rounding of x_in
    a = np.empty((len(live), Hq, D))
    for b in range(B):
        sel = np.nonzero(bat == b)[0]
        a[sel] = attention_rows(q[sel], kco[b], np.abs(vco[b]))
    a = a.reshape(len(live), d)
    bound = 2.0 ** -7 * (a + np.abs(want)) + 2.0 ** -8 * np.abs(x64) + 1e-6
    assert_within(got, want, bound, f"{name}: attention output element-wise")
    # fresh cache rows and the untouched ones
    written = np.zeros((B, S), dtype=bool)
    written[bat, pos] = True
    kg = np64(kcg)
    assert_close(kg[written], kco[written], 2e-2, f"{name}: fresh K rows")
    assert np.array_equal(kg[~written], kc[~written])
