"""Transformer pieces of the oracle (test infrastructure).

The pages name the model family (LLaDA-8B, Dream-7B: bidirectional, i.e.
non-causal, masked-diffusion transformers; ES-dLLM summary section 1) but no
layer internals.  The plain reading used here: pre-norm blocks without
biases, RMSNorm, rotate-half RoPE on Q and K at absolute positions,
grouped-query attention with scale 1/sqrt(D) and no mask, SwiGLU FFN.

Two independent forms are kept on purpose:
* ``layer_rows`` runs one layer on an arbitrary subset of rows and attends
  over persistent per-layer K/V caches -- the partial update of ES-dLLM
  (technical summary 2.1 item 2: only selected positions run attention and
  FFN, skipped positions reuse cached K/V/hidden) and SureLock (2.1 items 2-3:
  locked rows skip the computation but stay attendable via cached K/V).
* ``dense_forward`` recomputes every position of every layer with no caches
  and no row lists; with all rows active the partial update must equal it.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_bf16


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE.  x: [R, H, D]; pos: [R] absolute positions.

    For j < D/2 with theta_j = base^(-2j/D) and angle a = pos * theta_j:
    (x_j, x_{j+D/2}) -> (x_j cos a - x_{j+D/2} sin a, x_{j+D/2} cos a + x_j sin a).
    """
    D = x.shape[-1]
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * j / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]      # [R, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x), written to avoid overflow of exp for large |x|."""
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = x[pos] / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = x[~pos] * ex / (1.0 + ex)
    return out


LOG2E = 1.4426950408889634   # log2(e)


def attention_rows(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, p_store=None) -> np.ndarray:
    """Bidirectional attention of R queries over all S cached keys of one sequence.

    q: [R, Hq, D]; k_cache, v_cache: [S, Hkv, D]; query head h reads KV head
    h // (Hq / Hkv).  Every key is visible (no causal mask).  Returns [R, Hq, D].

    ``p_store`` (bf16 storage mode) is the rounding of the softmax weights that multiply V: the
    GPU holds them in bf16 as the matrix-core operand.  They are taken as w_j = 2^(x_j - M) with
    x_j = s_j log2(e) and M = ceil(max_j x_j): scaling by a power of two leaves a value's bf16
    rounding unchanged, so the rounded weights are the same against any integer reference a
    kernel may use (and however it splits the keys).  The output is sum_j p_store(w_j) V_j over
    the unrounded sum_j w_j.  Without ``p_store`` the weights stay exact (plain softmax).
    """
    R, Hq, D = q.shape
    S, Hkv, _ = k_cache.shape
    g = Hq // Hkv
    out = np.empty((R, Hq, D), dtype=np.float64)
    scale = 1.0 / np.sqrt(D)
    for h in range(Hq):
        kh = k_cache[:, h // g, :]                       # [S, D]
        vh = v_cache[:, h // g, :]
        s = (q[:, h, :] @ kh.T) * scale                  # [R, S]
        if p_store is None:
            s = s - np.max(s, axis=1, keepdims=True)
            p = np.exp(s)
            p = p / np.sum(p, axis=1, keepdims=True)
            out[:, h, :] = p @ vh
        else:
            x = s * LOG2E
            w = np.exp2(x - np.ceil(np.max(x, axis=1, keepdims=True)))
            out[:, h, :] = (p_store(w) @ vh) / np.sum(w, axis=1, keepdims=True)
    return out


def layer_rows(lw: dict, x_rows: np.ndarray, pos: np.ndarray, batch: np.ndarray,
               k_cache: np.ndarray, v_cache: np.ndarray, *, n_heads: int, n_kv_heads: int,
               rope_base: float, eps: float, store) -> np.ndarray:
    """One transformer layer on a subset of rows (the partial update).

    x_rows: [R, d] residual stream of the active rows; pos/batch: [R] position
    and sequence of each row.  k_cache/v_cache: [B, S, Hkv, D], updated in
    place at (batch, pos) of the active rows *before* attention; all other
    cache rows are left as they are and are attended as-is.  ``store`` rounds
    at the storage points.  Returns the new residual stream of the rows.
    """
    R, d = x_rows.shape
    D = k_cache.shape[-1]
    Hq, Hkv = n_heads, n_kv_heads
    n = store(rmsnorm(x_rows, lw["attn_norm"], eps))
    q = (n @ lw["wq"].T).reshape(R, Hq, D)
    k = (n @ lw["wk"].T).reshape(R, Hkv, D)
    v = (n @ lw["wv"].T).reshape(R, Hkv, D)
    q = store(rope(q, pos, rope_base))
    k = store(rope(k, pos, rope_base))
    v = store(v)
    k_cache[batch, pos] = k
    v_cache[batch, pos] = v
    o = np.empty((R, Hq, D), dtype=np.float64)
    p_store = store if store is round_bf16 else None   # bf16 softmax weights in bf16 storage mode
    for b in np.unique(batch):
        sel = np.nonzero(batch == b)[0]
        o[sel] = attention_rows(q[sel], k_cache[b], v_cache[b], p_store)
    o = store(o.reshape(R, Hq * D))
    x = store(x_rows + o @ lw["wo"].T)
    n2 = store(rmsnorm(x, lw["ffn_norm"], eps))
    gate = n2 @ lw["wg"].T
    up = n2 @ lw["wu"].T
    h = store(silu(gate) * up)
    x = store(x + h @ lw["wd"].T)
    return x


def lm_logits(h_rows: np.ndarray, final_norm: np.ndarray, lm_head: np.ndarray, eps: float, store) -> np.ndarray:
    """Logits of the given rows: rmsnorm(h) * g_f @ W_lm^T, stored as fp32."""
    from .numerics import fl32
    n = store(rmsnorm(h_rows, final_norm, eps))
    return fl32(n @ lm_head.T)


def dense_forward(weights: dict, tokens: np.ndarray, *, n_heads: int, n_kv_heads: int,
                  rope_base: float, eps: float, store, boundary_layer: int | None = None) -> dict:
    """Full recompute of every position at every layer (no caches, no row lists).

    tokens: [B, S].  Returns the per-layer K/V ([L] of [B, S, Hkv, D]), the
    hidden state entering ``boundary_layer`` (if given), the final hidden
    state [B, S, d] and the fp32 logits [B, S, V].
    """
    B, S = tokens.shape
    E = weights["embed"]
    d = E.shape[1]
    x = E[tokens.reshape(-1)].reshape(B, S, d).copy()
    Hq, Hkv = n_heads, n_kv_heads
    pos = np.arange(S)
    ks, vs = [], []
    h_bnd = None
    L = len(weights["layers"])
    for l, lw in enumerate(weights["layers"]):
        if boundary_layer is not None and l == boundary_layer:
            h_bnd = x.copy()
        D = lw["wq"].shape[0] // Hq
        g = Hq // Hkv
        n = store(rmsnorm(x, lw["attn_norm"], eps))
        q = store(np.stack([rope((n[b] @ lw["wq"].T).reshape(S, Hq, D), pos, rope_base) for b in range(B)]))
        k = store(np.stack([rope((n[b] @ lw["wk"].T).reshape(S, Hkv, D), pos, rope_base) for b in range(B)]))
        v = store(np.stack([(n[b] @ lw["wv"].T).reshape(S, Hkv, D) for b in range(B)]))
        ks.append(k.copy())
        vs.append(v.copy())
        o = np.empty((B, S, Hq, D))
        for b in range(B):
            for h in range(Hq):
                sc = q[b, :, h, :] @ k[b, :, h // g, :].T / np.sqrt(D)     # [S, S], no mask
                if store is round_bf16:   # bf16 weights against a power-of-two reference
                    xl = sc * LOG2E
                    w = np.exp2(xl - np.ceil(xl.max(axis=1, keepdims=True)))
                    o[b, :, h, :] = (store(w) @ v[b, :, h // g, :]) / w.sum(axis=1, keepdims=True)
                else:
                    w = np.exp(sc - sc.max(axis=1, keepdims=True))
                    w /= w.sum(axis=1, keepdims=True)
                    o[b, :, h, :] = w @ v[b, :, h // g, :]
        o = store(o.reshape(B, S, Hq * D))
        x = store(x + o @ lw["wo"].T)
        n2 = store(rmsnorm(x, lw["ffn_norm"], eps))
        a = n2 @ lw["wg"].T
        u = n2 @ lw["wu"].T
        x = store(x + store(a / (1.0 + np.exp(-a)) * u) @ lw["wd"].T)
    if boundary_layer is not None and boundary_layer == L:
        h_bnd = x.copy()
    logits = lm_logits(x.reshape(B * S, d), weights["final_norm"], weights["lm_head"], eps, store)
    return {"k": ks, "v": vs, "h_bnd": h_bnd, "h_fin": x, "logits": logits.reshape(B, S, -1)}
