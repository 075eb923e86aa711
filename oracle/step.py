"""One token-skipping denoising iteration, step by step (test infrastructure).

Order of operations (ES-dLLM technical summary 2.1; SureLock 2.1):
  1. embed the current tokens;
  2. run layers below the boundary b on every position (on a full step, every
     layer runs on every position);
  3. at layer b, score every position from the previous iteration's
     confidence (or KL) and the change of the hidden state entering layer b
     since the previous iteration (Eq. 1), keep that hidden state for the next
     iteration, and select the active rows;
  4. run layers b..L-1 on the active rows only: their fresh K/V overwrite the
     cache rows, and they attend over the whole cache, so skipped positions
     contribute the K/V cached when they were last computed;
  5. write the active rows' final hidden state, run the LM head on them and
     compute confidence, argmax and local KL; skipped positions keep all of
     their previous statistics;
  6. SureLock lock update and/or unmasking of the current block (by
     confidence, or the positions a dilated schedule plans for this round).

Nested boundaries (ES-dLLM technical summary 2.1 item 2 selects at the start of
a layer with a per-layer score I_{l,i}): optionally, at later layers
n_1 < n_2 < ... the active rows are scored again, from the change of the hidden
state entering that layer since it was last computed for the row (a per-layer
cache, filled by full steps and updated for every row that reaches the layer),
and only the top k_j of them continue.  A row dropped at layer n_j keeps the
K/V it wrote below n_j; from n_j on it is skipped like any other row (cached
K/V, final hidden state and statistics reused).

Per-layer caching (dLLM-Cache summary section 3, f2): with layer_cache set, every layer
l >= b runs a partial update instead of the single selection at b.  Entering layer l, each
row's hidden state is compared with the one it had when the row was last computed at l (a
per-layer input cache); the top k rows of each sequence by the step's score settings
(alpha 0 and the cosine change term give the feature-similarity test) are computed through
the layer, their K/V overwrite the cache rows, and every other row takes the output it had
when it was last computed at l (a per-layer output cache).  Both caches keep the new values of
the computed rows.  A full step computes every row at every layer and fills both caches.  The
long-interval prompt cache is the caller's force == 2 on prompt positions between full steps.
After the last layer the rows computed there get the LM head; all others keep their
statistics (their final hidden state is the cached one).  The compared feature is the row's hidden
state entering the layer, or (cache_feature "value") the layer's V projection of that input
against the V the row holds in the layer's K/V cache, i.e. the V computed when the row was last
computed there: the V projection of every row is the extra cost of this test.

Readings where the pages leave a step open: the mask id is the last vocabulary
entry and is excluded from softmax and argmax; a locked row (force == 2) skips
every layer and the LM head, its cached K/V stay attendable; step 0 has no
previous posterior, so its KL is +inf; a nested selection is a top-k with the
step's score settings (alpha, change term), forced rows kept first.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .importance import VAR_L1N, importance_score
from .numerics import store_fn
from .post import surelock_update, unmask_forced, unmask_topn
from .selection import FORCE_EXCLUDED, select_thresh_cap, select_topk
from .transformer import layer_rows, lm_logits, rmsnorm
from .vocab import conf_kl, kl_state_value

SEL_TOPK, SEL_THRESH_CAP, SEL_UNLOCKED = 0, 1, 2
UNMASK_CONF, UNMASK_FORCED = 0, 1


@dataclass
class OracleModel:
    weights: dict
    n_heads: int
    n_kv_heads: int
    mask_id: int
    mode: str = "bf16"
    rope_base: float = 10000.0
    eps: float = 1e-5

    @property
    def n_layers(self) -> int:
        return len(self.weights["layers"])


@dataclass
class ScoreCfg:
    alpha: float = 0.5
    conf_inverted: bool = False
    var: int = VAR_L1N
    sel: int = SEL_TOPK
    k: int = 1
    tau: float = 0.0


@dataclass
class StepCfg:
    boundary_layer: int
    full_step: bool
    score: ScoreCfg = field(default_factory=ScoreCfg)
    lock_kl_eps: float = -1.0      # < 0 disables locking
    lock_conf_min: float = 0.9
    unmask_n: int = 0
    block_lo: int = 0
    block_hi: int = 0
    unmask_mode: int = UNMASK_CONF
    nested: tuple = ()             # ((layer, k), ...): later layers that narrow the active set
    layer_cache: bool = False      # per-layer partial update from layer b on (dLLM-Cache)
    cache_feature: str = "hidden"  # what the layer cache compares: "hidden" (the layer input) or "value"


@dataclass
class OracleState:
    tokens: np.ndarray
    k_cache: list
    v_cache: list
    h_bnd_prev: np.ndarray | None
    h_fin: np.ndarray
    conf: np.ndarray
    kl: np.ndarray
    argmax: np.ndarray
    logits_prev: np.ndarray | None
    force: np.ndarray
    have_prev: bool = False
    kl_state_bf16: bool = False  # previous logits kept rounded to bf16 (compact KL state)
    h_nested: list = field(default_factory=list)  # per nested boundary: [B, S, d] hidden state entering it
    x_in: list = field(default_factory=list)      # per layer (layer cache): [B, S, d] input when last computed
    x_out: list = field(default_factory=list)     # per layer (layer cache): [B, S, d] output when last computed

    def copy(self) -> "OracleState":
        return OracleState(
            self.tokens.copy(), [k.copy() for k in self.k_cache], [v.copy() for v in self.v_cache],
            None if self.h_bnd_prev is None else self.h_bnd_prev.copy(), self.h_fin.copy(),
            self.conf.copy(), self.kl.copy(), self.argmax.copy(),
            None if self.logits_prev is None else self.logits_prev.copy(), self.force.copy(), self.have_prev,
            self.kl_state_bf16, [h.copy() for h in self.h_nested], [h.copy() for h in self.x_in],
            [h.copy() for h in self.x_out])


def new_state(model: OracleModel, tokens: np.ndarray, track_kl: bool, kl_state_bf16: bool = False,
              n_nested: int = 0, layer_cache: bool = False) -> OracleState:
    B, S = tokens.shape
    w = model.weights
    d = w["embed"].shape[1]
    V = w["embed"].shape[0]
    D = w["layers"][0]["wq"].shape[0] // model.n_heads
    Hkv = model.n_kv_heads
    L = model.n_layers
    return OracleState(
        tokens=np.array(tokens, dtype=np.int64),
        k_cache=[np.zeros((B, S, Hkv, D)) for _ in range(L)],
        v_cache=[np.zeros((B, S, Hkv, D)) for _ in range(L)],
        h_bnd_prev=None,
        h_fin=np.zeros((B, S, d)),
        conf=np.zeros((B, S)),
        kl=np.full((B, S), np.inf),
        argmax=np.zeros((B, S), dtype=np.int64),
        logits_prev=np.zeros((B * S, V)) if track_kl else None,
        force=np.zeros((B, S), dtype=np.uint8),
        kl_state_bf16=kl_state_bf16,
        h_nested=[np.zeros((B, S, d)) for _ in range(n_nested)],
        x_in=[np.zeros((B, S, d)) for _ in range(L)] if layer_cache else [],
        x_out=[np.zeros((B, S, d)) for _ in range(L)] if layer_cache else [],
    )


def _select(scfg: ScoreCfg, scores: np.ndarray, force: np.ndarray) -> np.ndarray:
    if scfg.sel == SEL_TOPK:
        return select_topk(scores, force, scfg.k)
    if scfg.sel == SEL_THRESH_CAP:
        return select_thresh_cap(scores, force, scfg.tau, scfg.k)
    if scfg.sel == SEL_UNLOCKED:
        return select_topk(scores, force, len(scores))
    raise ValueError(f"unknown selection mode {scfg.sel}")


def skip_step(model: OracleModel, st: OracleState, cfg: StepCfg) -> tuple[OracleState, dict]:
    """Run one iteration; returns the new state and {"rows", "scores"}."""
    st = st.copy()
    store = store_fn(model.mode)
    w = model.weights
    B, S = st.tokens.shape
    d = w["embed"].shape[1]
    L = model.n_layers
    b_lay = int(cfg.boundary_layer)
    if not (0 <= b_lay <= L):
        raise ValueError("boundary layer out of range")
    full = bool(cfg.full_step)
    lcache = bool(cfg.layer_cache)
    if lcache:
        if b_lay >= L:
            raise ValueError("the layer cache needs a layer at or above the boundary")
        if len(st.x_in) != L or len(st.x_out) != L:
            raise ValueError("a layer-cache step needs the per-layer caches in the state")
        if cfg.nested:
            raise ValueError("nested boundaries and the layer cache do not combine")
        if not full and not st.have_prev:
            raise ValueError("a sparse layer-cache step needs caches filled by an earlier step")
        if cfg.cache_feature not in ("hidden", "value"):
            raise ValueError(f"unknown layer-cache feature {cfg.cache_feature!r}")
    elif not full and st.h_bnd_prev is None:
        raise ValueError("a sparse step needs the previous boundary hidden state")
    nested = [(int(nl), int(nk)) for nl, nk in cfg.nested]
    if len(nested) > len(st.h_nested):
        raise ValueError("the state holds fewer nested caches than the step names")
    prev_layer = b_lay
    for nl, nk in nested:
        if not (prev_layer < nl < L) or nk < 0:
            raise ValueError("nested layers must increase strictly after the boundary, below L; k >= 0")
        prev_layer = nl

    x = w["embed"][st.tokens.reshape(-1)].reshape(B * S, d).copy()
    rows = np.arange(B * S)                   # flat b*S + i of the rows being computed
    scores = None
    h_bnd_new = None

    def boundary():
        nonlocal rows, x, scores, h_bnd_new
        h_bnd_new = x.reshape(B, S, d).copy()
        if full:
            return
        s = importance_score(x, st.h_bnd_prev.reshape(B * S, d), st.conf.reshape(-1), st.kl.reshape(-1),
                             alpha=cfg.score.alpha, var=cfg.score.var, conf_inverted=cfg.score.conf_inverted)
        scores = s.reshape(B, S)
        sel = [b * S + _select(cfg.score, scores[b], st.force[b]) for b in range(B)]
        rows = np.concatenate(sel).astype(np.int64)
        x = x[rows].copy()

    nested_rows, nested_scores = [], []

    def nested_boundary(j, k):
        nonlocal rows, x
        hn = st.h_nested[j].reshape(B * S, d)
        if full:
            hn[rows] = x
            return
        s = importance_score(x, hn[rows], st.conf.reshape(-1)[rows], st.kl.reshape(-1)[rows],
                             alpha=cfg.score.alpha, var=cfg.score.var, conf_inverted=cfg.score.conf_inverted)
        hn[rows] = x            # the hidden state entering this layer, kept for the next iteration
        nested_scores.append((rows.copy(), s.copy()))
        keep = []
        for b in range(B):
            in_b = (rows // S) == b
            pos = rows[in_b] % S
            sc = np.zeros(S)
            sc[pos] = s[in_b]
            fo = np.full(S, FORCE_EXCLUDED, dtype=np.uint8)   # only the active rows compete
            fo[pos] = np.minimum(st.force[b, pos], 1)
            keep.append(b * S + select_topk(sc, fo, k))
        new_rows = np.concatenate(keep).astype(np.int64)
        x = x[np.searchsorted(rows, new_rows)].copy()
        rows = new_rows
        nested_rows.append(rows.copy())

    layer_sel, layer_scores = [], []

    def cached_layer(l, lw):
        """Partial update of layer l over every row (x: all B*S rows in, all rows out)."""
        nonlocal x, rows
        xi, xo = st.x_in[l].reshape(B * S, d), st.x_out[l].reshape(B * S, d)
        if full:
            xi[:] = x
            x = layer_rows(lw, x, rows % S, rows // S, st.k_cache[l], st.v_cache[l], n_heads=model.n_heads,
                           n_kv_heads=model.n_kv_heads, rope_base=model.rope_base, eps=model.eps, store=store)
            xo[:] = x
            return
        if cfg.cache_feature == "value":
            # the layer's V projection of every row's current input against the V cached when the
            # row was last computed at this layer (its rows of the layer's V cache)
            v_new = store(store(rmsnorm(x, lw["attn_norm"], model.eps)) @ lw["wv"].T)
            feat, feat_prev = v_new, st.v_cache[l].reshape(B * S, -1)
        else:
            feat, feat_prev = x, xi
        s = importance_score(feat, feat_prev, st.conf.reshape(-1), st.kl.reshape(-1), alpha=cfg.score.alpha,
                             var=cfg.score.var, conf_inverted=cfg.score.conf_inverted).reshape(B, S)
        sel = np.concatenate([b * S + _select(cfg.score, s[b], st.force[b]) for b in range(B)]).astype(np.int64)
        layer_scores.append(s)
        layer_sel.append(sel)
        xi[sel] = x[sel]
        xo[sel] = layer_rows(lw, x[sel], sel % S, sel // S, st.k_cache[l], st.v_cache[l], n_heads=model.n_heads,
                             n_kv_heads=model.n_kv_heads, rope_base=model.rope_base, eps=model.eps, store=store)
        x = xo.copy()
        rows = sel

    for l in range(L):
        if l == b_lay and not lcache:
            boundary()
        for j, (nl, nk) in enumerate(nested):
            if l == nl:
                nested_boundary(j, nk)
        lw = w["layers"][l]
        if lcache and l >= b_lay:
            cached_layer(l, lw)
            continue
        x = layer_rows(lw, x, rows % S, rows // S, st.k_cache[l], st.v_cache[l],
                       n_heads=model.n_heads, n_kv_heads=model.n_kv_heads,
                       rope_base=model.rope_base, eps=model.eps, store=store)
    if b_lay == L and not lcache:
        boundary()

    if not lcache:
        st.h_bnd_prev = h_bnd_new
    if x.shape[0] != len(rows):          # layer cache: x holds every row, the last layer computed `rows`
        x = x[rows]
    hf = st.h_fin.reshape(B * S, d)
    hf[rows] = x
    z = lm_logits(x, w["final_norm"], w["lm_head"], model.eps, store)
    zp = None if (st.logits_prev is None or not st.have_prev) else st.logits_prev[rows]
    conf, arg, kl = conf_kl(z, zp, model.mask_id, st.kl_state_bf16)
    st.conf.reshape(-1)[rows] = conf
    st.argmax.reshape(-1)[rows] = arg
    st.kl.reshape(-1)[rows] = kl
    if st.logits_prev is not None:
        st.logits_prev[rows] = kl_state_value(z, st.kl_state_bf16)
    if cfg.lock_kl_eps >= 0:
        st.force = surelock_update(st.force.reshape(-1), rows, st.conf.reshape(-1), st.kl.reshape(-1),
                                   st.have_prev, cfg.lock_kl_eps, cfg.lock_conf_min).reshape(B, S)
    if cfg.unmask_n > 0:
        if cfg.unmask_mode == UNMASK_FORCED:
            st.tokens = unmask_forced(st.tokens, st.force, st.argmax, model.mask_id, cfg.block_lo, cfg.block_hi)
        else:
            st.tokens = unmask_topn(st.tokens, st.conf, st.argmax, model.mask_id,
                                    cfg.block_lo, cfg.block_hi, cfg.unmask_n)
    st.have_prev = True
    return st, {"rows": rows, "scores": scores, "logits": z, "nested_rows": nested_rows,
                "nested_scores": nested_scores, "layer_rows": layer_sel, "layer_scores": layer_scores}
