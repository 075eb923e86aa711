/*
 * dllm.h -- C ABI of libdllm: one token-skipping denoising iteration of a
 * bidirectional masked-diffusion transformer on an MI355X (gfx950).
 *
 * Method sources (cited by page title and section):
 *  [ES]  "ES-dLLM: Efficient Inference for Diffusion Large Language Models by
 *        Early-Skipping", gist.science summary, technical summary section 2.1
 *        (item 1: importance score, Eq. 1; item 2: partial cache update and
 *        early skip) and section 2.2 (periodic refresh).
 *  [SL]  "Stopping Computation for Converged Tokens in Masked Diffusion-LM
 *        Decoding" (SureLock), gist.science summary, technical summary
 *        section 2.1 (items 1-4: local-KL lock rule, skipped Q-projection and
 *        FFN, cached K/V stay attendable, O(M_t N d) cost).
 *  [DC]  dLLM-Cache explainer (aibr.jp), section 3 (similarity-gated partial
 *        response update, long-interval prompt cache) and section 4 (update
 *        ratio rho).
 *  [DUS] "Plan for Speed: Dilated Scheduling for Masked Diffusion Language
 *        Models", gist.science summary, technical summary section 2.
 *
 * Conventions shared by every entry point
 *  - All pointers named in a struct or argument list as "device" are device
 *    pointers on the current HIP device; "host" pointers are read during the
 *    call only.  The library never allocates, frees or retains memory: the
 *    caller owns every buffer.  Device buffers must be 16-byte aligned.
 *  - Matrices are row-major.  Weights use the nn.Linear layout [out, in].
 *  - Element type (dllm_dtype) applies to weights, activations and K/V caches;
 *    logits, scores, confidence and KL are always fp32.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued on it and the call returns without synchronising.
 *  - Every function returns a dllm_status.  Arguments are validated on the
 *    host before any launch; on error nothing is launched.  DLLM_ELAUNCH
 *    reports a failed kernel launch.  Faults inside kernels surface at the
 *    caller's next synchronisation.  Device-resident indices and token ids
 *    are preconditions (token ids outside [0, V) are clamped).
 *  - Row layout of "active" buffers: padded per sequence.  Row r = b*k_max + j
 *    holds the j-th active position of sequence b when j < n_active[b]; rows
 *    with j >= n_active[b] are dead and their contents are unspecified.
 *  - Calls on one stream are ordered; calls that share a workspace or state
 *    must not overlap on different streams.
 *  - bf16 shapes: d, n_heads * head_dim and d_ff are multiples of 64,
 *    head_dim is 128, and the kernels address memory with 32-bit offsets, so
 *    the SwiGLU weight ((d_ff + 128) x d elements), 256 rows of any GEMM input
 *    and one sequence's K/V cache of one layer (S x n_kv_heads x 128) must each
 *    stay under 2 GiB; other shapes return DLLM_ESHAPE before any launch.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DLLM_OK = 0,
  DLLM_EINVAL = 1,     /* bad argument (NULL pointer, out-of-range value) */
  DLLM_ESHAPE = 2,     /* unsupported or inconsistent shape */
  DLLM_EDTYPE = 3,     /* unknown dtype */
  DLLM_EWORKSPACE = 4, /* workspace missing or smaller than required */
  DLLM_ELAUNCH = 5     /* a kernel launch failed */
} dllm_status;

typedef enum { DLLM_F32 = 0, DLLM_BF16 = 1 } dllm_dtype;

/* Change term of the importance score ([ES] Eq. 1 and variants). */
typedef enum {
  DLLM_VAR_L1N = 0,   /* ||Hc-Hp||_1 / (sqrt(w) ||Hp||_2)      [ES] Eq. 1 */
  DLLM_VAR_COS = 1,   /* 1 - cos(Hc, Hp) = 0.5 || Hc/|Hc| - Hp/|Hp| ||^2  [DC] sec. 3 */
  DLLM_VAR_L2REL = 2, /* ||Hc-Hp||_2 / ||Hp||_2 */
  DLLM_VAR_KL = 3,    /* previous step's local KL              [SL] 2.1 item 1 */
  DLLM_VAR_NONE = 4   /* 0 */
} dllm_var;

/* Active-row selection ([ES] 2.1 item 2; [DC] sec. 3-4; [SL] 2.1 item 2). */
typedef enum {
  DLLM_SEL_TOPK = 0,       /* the k best candidates */
  DLLM_SEL_THRESH_CAP = 1, /* forced rows and rows scoring > tau, capped at k */
  DLLM_SEL_UNLOCKED = 2    /* every candidate (SureLock compaction) */
} dllm_sel;

/* How a step unmasks positions of [block_lo, block_hi) (with unmask_n > 0). */
typedef enum {
  DLLM_UNMASK_CONF = 0,   /* the unmask_n most confident masked positions (ES-dLLM sec. 1) */
  DLLM_UNMASK_FORCED = 1  /* every masked position with force == DLLM_FORCE_ON: the positions a
                             dilated schedule plans for this round ([DUS] sec. 2) */
} dllm_unmask_mode;

/* dllm_step_cfg.layer_cache: what each cached layer compares to pick the rows it recomputes
 * ([DC] section 3: a partial response update decided by feature-vector similarity). */
typedef enum {
  DLLM_LCACHE_OFF = 0,
  DLLM_LCACHE_HIDDEN = 1, /* the hidden state entering the layer, against x_in_cache[l] */
  DLLM_LCACHE_VALUE = 2   /* the layer's V projection of that input (every unlocked position), against
                             the V the position holds in the layer's V cache */
} dllm_layer_cache_mode;

/* Most nested boundaries a step may name (dllm_step_cfg.nested_layer). */
#define DLLM_MAX_NESTED 3

/* force[] values: per position. */
enum { DLLM_FORCE_NONE = 0, DLLM_FORCE_ON = 1, DLLM_FORCE_EXCLUDED = 2 };

typedef struct {
  int32_t B, S;                 /* sequences, positions per sequence */
  int32_t d;                    /* hidden size */
  int32_t n_heads, n_kv_heads;  /* query heads, K/V heads (GQA group = n_heads/n_kv_heads) */
  int32_t head_dim;             /* D (128, or 64 for the fp32 path) */
  int32_t d_ff;                 /* SwiGLU width F */
  int32_t vocab;                /* V */
  int32_t n_layers;             /* L */
} dllm_dims;

typedef struct {
  const void *attn_norm;  /* device [d] */
  const void *w_qkv;      /* device [(Hq + 2 Hkv) D, d]: Q rows, then K rows, then V rows */
  const void *w_o;        /* device [d, Hq D] */
  const void *ffn_norm;   /* device [d] */
  const void *w_gate_up;  /* device [2F, d]: gate rows, then up rows */
  const void *w_down;     /* device [d, F] */
  /* Optional second copies in MFMA fragment order (dllm_pack_weight), or NULL.  When present,
   * the bf16 QKV, gate/up and down products over at most 128 active rows stream them straight
   * into registers instead of the row-major copies above (which stay in use for every other
   * product), whenever the packed planner (dllm_packed_plan) covers the shape: N a multiple of
   * 64, K a multiple of 64 with at least 6-7 stages of 64 per K split (the LLaDA-8B and Dream-7B
   * shapes are covered).  The O product keeps its row-major tiles (its 4096 x 4096 weight is too
   * short a stream per workgroup for the packed form to pay). */
  const void *w_gate_up_packed; /* w_gate_up packed with gate/up interleave F */
  const void *w_down_packed;    /* w_down packed without interleave */
  const void *w_qkv_packed;     /* w_qkv packed without interleave */
} dllm_layer_w;

typedef struct {
  dllm_dims dims;
  int32_t dtype;                 /* dllm_dtype */
  float rope_base;               /* rotate-half RoPE base (1e4) */
  float rms_eps;                 /* RMSNorm epsilon (1e-5) */
  int32_t mask_id;               /* mask token; excluded from softmax/argmax */
  const void *embed;             /* device [V, d] */
  const dllm_layer_w *layers;    /* host array [L] */
  const void *final_norm;        /* device [d] */
  const void *lm_head;           /* device [V, d] */
  /* Optional second copy of lm_head in MFMA fragment order (dllm_pack_weight, no interleave), or
   * NULL.  When present, the bf16 LM head over at most 128 computed rows streams it into
   * registers (one K split: the vocabulary pass reads whole logits) whenever V is a multiple of
   * 64 and d of 64; every other LM head product keeps the row-major copy.  Same logits up to the
   * fp32 summation order. */
  const void *lm_head_packed;
} dllm_model;

typedef struct {
  float alpha;            /* weight of the confidence term ([ES] Eq. 1) */
  int32_t conf_inverted;  /* 0: phi(c) = c as in Eq. 1;  1: phi(c) = 1 - c */
  int32_t var;            /* dllm_var */
  int32_t sel;            /* dllm_sel */
  int32_t k;              /* rows kept per sequence (cap for THRESH_CAP) */
  float tau;              /* THRESH_CAP threshold (score > tau qualifies) */
} dllm_score_cfg;

/* Persistent per-run state.  The library reads and writes the device arrays
 * and flips bnd_cur / sets have_prev in this host struct. */
typedef struct {
  int32_t *tokens;        /* device [B, S] token ids (in/out: unmasking writes them) */
  void **k_cache;         /* host array [L] of device [B, S, Hkv, D] */
  void **v_cache;         /* host array [L] of device [B, S, Hkv, D] */
  void *h_bnd[2];         /* device [B, S, d] x2: hidden state entering the boundary layer */
  int32_t bnd_cur;        /* index of h_bnd holding the previous step's state */
  void *h_fin;            /* device [B, S, d] final hidden state */
  float *conf;            /* device [B, S] max softmax probability */
  float *kl;              /* device [B, S] local KL (+inf before a previous posterior exists) */
  int32_t *argmax;        /* device [B, S] most likely non-mask token */
  void *logits_prev;      /* device [B*S, V] previous logits in logits_prev_dtype, or NULL (then KL is
                             not tracked) */
  uint8_t *force;         /* device [B, S] dllm_force values, or NULL (all 0) */
  int32_t *idx;           /* device [B, k_max] out: active positions (ascending, -1 padded) */
  int32_t *n_active;      /* device [B] out */
  int32_t k_max;          /* row stride of idx and of the active-row buffers (1..S); a full
                             step leaves idx / n_active unchanged */
  int32_t have_prev;      /* 0 until the first step has run */
  int32_t logits_prev_dtype; /* DLLM_F32, or DLLM_BF16 for the compact KL state: the previous logits
                             are stored rounded to bf16 (RNE) and the KL compares the bf16-rounded
                             current logits with them, so identical logits still give KL = 0;
                             conf and argmax always come from the fp32 logits */
  void *h_nested[DLLM_MAX_NESTED]; /* device [B, S, d] each, or NULL: the hidden state entering
                             nested layer j the last time each position was computed there
                             (written by full steps and by every row reaching that layer) */
  void **x_in_cache;      /* per-layer cache (step cfg layer_cache), or NULL: host array [L] of device
                             [B, S, d], the hidden state entering layer l when each position was last
                             computed there; entries below the boundary layer may be NULL */
  void **x_out_cache;     /* the same for the hidden state leaving layer l */
} dllm_state;

/* Kernel classes the measurement hook can bracket. */
typedef enum {
  DLLM_TK_NONE = 0,
  DLLM_TK_QKV = 1,      /* QKV product of a layer */
  DLLM_TK_ATTN = 2,     /* bidirectional attention of a layer */
  DLLM_TK_O = 3,        /* output projection of a layer */
  DLLM_TK_FFN_UP = 4,   /* gate/up product with the SwiGLU epilogue */
  DLLM_TK_FFN_DOWN = 5, /* down projection of a layer */
  DLLM_TK_LM_HEAD = 6,  /* LM-head product */
  DLLM_TK_VOCAB = 7,    /* confidence / argmax / KL vocabulary pass */
  DLLM_TK_SCORE = 8,    /* importance scores */
  DLLM_TK_SELECT = 9    /* active-row selection */
} dllm_timed_kernel;

typedef struct {
  int32_t kernel;     /* dllm_timed_kernel to bracket */
  int32_t max_rows;   /* only launches whose row capacity is <= max_rows (0: all) */
  int32_t capacity;   /* number of event pairs in start/stop */
  int32_t count;      /* out: event pairs recorded so far (the caller resets it) */
  void **start;       /* host array [capacity] of caller-created hipEvent_t */
  void **stop;        /* host array [capacity] of caller-created hipEvent_t */
} dllm_timing;

typedef struct {
  int32_t boundary_layer;   /* b: layers < b run on all rows; 0 <= b <= L */
  int32_t full_step;        /* 1: every layer on every row (first step, refresh) */
  dllm_score_cfg score;
  float lock_kl_eps;        /* SureLock epsilon; < 0 disables locking */
  float lock_conf_min;      /* lock also requires conf > this */
  int32_t unmask_n;         /* unmask this many masked positions per sequence (0: none) */
  int32_t block_lo, block_hi; /* unmasking window [lo, hi) */
  int32_t unmask_mode;      /* dllm_unmask_mode */
  void *ws;                 /* device workspace */
  size_t ws_bytes;
  /* Nested boundaries ([ES] 2.1 item 2: selection at the start of a layer with the per-layer
   * score I_{l,i}).  At layers boundary_layer < nested_layer[0] < ... < L the rows still active
   * are scored again with `score`'s alpha / change term, the change taken between the hidden state
   * entering that layer and state->h_nested[j] at the row's position; the top nested_k[j] of
   * them (forced rows first, ties to the lower position) continue, the others are skipped from
   * that layer on (they keep the K/V written below it; their final hidden state and statistics
   * stay cached).  h_nested[j] is then updated for every row that reached the layer.  A full
   * step fills h_nested[j] for every row.  idx / n_active report the last set. */
  int32_t n_nested;                       /* 0..DLLM_MAX_NESTED */
  int32_t nested_layer[DLLM_MAX_NESTED];
  int32_t nested_k[DLLM_MAX_NESTED];      /* 0 <= k <= state->k_max */
  /* Per-layer cache ([DC] section 3: partial response update gated by feature similarity; the
   * long-interval prompt cache is force == 2 on prompt positions between full steps).  With
   * layer_cache != DLLM_LCACHE_OFF, every layer l >= boundary_layer replaces the single selection:
   * each position's feature is scored with `score` (alpha 0 and DLLM_VAR_COS give the
   * cosine-similarity test) -- DLLM_LCACHE_HIDDEN: its hidden state entering l against
   * x_in_cache[l]; DLLM_LCACHE_VALUE: the layer's V projection of that input, computed for every
   * unlocked position, against the V the position holds in v_cache[l] (written when it was last
   * computed there) -- the top score.k per sequence (forced first, locked excluded, ties to the
   * lower position) are computed through layer l and written to both caches and the K/V cache,
   * and every other position takes x_out_cache[l] as its output.  The rows computed at the last
   * layer get the LM head; idx / n_active report them.  A full step fills both caches of layers
   * >= boundary_layer for every position.  Needs n_nested = 0; values outside the enum return
   * DLLM_EINVAL. */
  int32_t layer_cache;      /* dllm_layer_cache_mode */
  /* Measurement hook for benchmarks, or NULL: each launch of the chosen kernel class made by
   * this call is bracketed by hipEventRecord(start[i]) / hipEventRecord(stop[i]) on the call's
   * stream, for i = count, count + 1, ... until capacity is reached; count is advanced as pairs
   * are recorded (the caller resets it).  The struct belongs to this call only, so calls on
   * other threads or streams are unaffected.  Not for use under stream capture.  A malformed
   * struct returns DLLM_EINVAL before any launch; a failed event record returns DLLM_ELAUNCH. */
  dllm_timing *timing;
} dllm_step_cfg;

/* Bytes of device workspace needed by dllm_skip_step / dllm_layer_sparse for
 * these dims and an active-row stride k_max.  Returns 0 on invalid input. */
size_t dllm_workspace_size(const dllm_dims *dims, int32_t dtype, int32_t k_max);

/* Importance scores and active-row selection ([ES] 2.1 items 1-2 and Eq. 1;
 * [DC] sec. 3-4; [SL] 2.1 items 1-2).
 *  h_cur, h_prev: device [B, S, width] (dtype)   -- current / previous tensor
 *  conf_prev, kl_prev: device [B, S] fp32 (kl_prev may be NULL unless var = KL)
 *  force: device [B, S] or NULL; FORCE_ON rows always come first, FORCE_EXCLUDED
 *         rows are never selected.
 *  score = alpha * phi(conf) + (1 - alpha) * psi, computed in fp32.
 *  Selection order: forced, then score descending (NaN last, -0 == +0), then
 *  lower index.  Outputs: score_out device [B, S] (may be NULL),
 *  idx_out device [B, k_max] ascending and -1 padded, n_active_out device [B].
 *  h_next: device [B, S, width] or NULL: receives a copy of h_cur.
 *  Requires cfg->k <= k_max, width % 8 == 0 (bf16) or % 4 == 0 (fp32). */
int dllm_score_select(const void *h_cur, const void *h_prev, void *h_next, int32_t dtype,
                      const float *conf_prev, const float *kl_prev, const uint8_t *force,
                      int32_t B, int32_t S, int32_t width, const dllm_score_cfg *cfg,
                      float *score_out, int32_t *idx_out, int32_t *n_active_out, int32_t k_max,
                      void *stream);

/* Gather active rows ([ES] 2.1 item 2: selected positions continue).
 *  src device [B, S, width] -> dst device [B*k_max, width] (padded rows). */
int dllm_gather_rows(const void *src, const int32_t *idx, const int32_t *n_active, int32_t B,
                     int32_t S, int32_t k_max, int32_t width, int32_t dtype, void *dst, void *stream);

/* Scatter active rows back ([ES] 2.1 item 2: in-place cache update).
 *  src device [B*k_max, width] -> dst device [B, S, width]; other rows untouched. */
int dllm_scatter_rows(const void *src, const int32_t *idx, const int32_t *n_active, int32_t B,
                      int32_t S, int32_t k_max, int32_t width, int32_t dtype, void *dst, void *stream);

/* One transformer layer on the active rows only ([ES] 2.1 item 2; [SL] 2.1
 * items 2-4): RMSNorm -> QKV GEMM -> RoPE at the rows' absolute positions ->
 * K/V written into the caches at (b, idx) -> bidirectional GQA attention of
 * the active queries over all S cached keys -> O GEMM + residual -> RMSNorm
 * -> SwiGLU FFN + residual.
 *  x_act: device [B*k_max, d] residual stream of the active rows (in/out).
 *  idx/n_active: as produced by dllm_score_select.
 *  k_cache/v_cache: device [B, S, Hkv, D] of this layer; only rows (b, idx)
 *  are written.  ws: dllm_workspace_size(dims, dtype, k_max) bytes. */
int dllm_layer_sparse(const dllm_model *model, int32_t layer, void *x_act, const int32_t *idx,
                      const int32_t *n_active, int32_t k_max, void *k_cache, void *v_cache,
                      void *ws, size_t ws_bytes, void *stream);

/* Bytes of the library-owned scratch array dllm_layer_sparse_noalloc works in (one per GPU). */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* dllm_layer_sparse without a workspace, for callers that cannot allocate device memory: code
 * under stream capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layout and result as dllm_layer_sparse (the same kernels and launch plans, so the outputs are
 * bit-identical), but its scratch -- the normalised rows, Q, the attention output, the SwiGLU
 * rows, split-K and split-KV partials and row positions of B * k_max active rows -- lives in a
 * file-scope device array of DLLM_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs
 * on holds until the process ends.  Enough for one LLaDA-8B-shaped layer (d 4096, 32 heads,
 * F 12288) at up to about 256 active rows; a shape that needs more returns DLLM_EWORKSPACE before
 * any launch.  Nothing is allocated or freed: the array's address on the current device is
 * resolved on the first call on that device (the stream must belong to the current device).
 * Every call on one GPU shares that GPU's array and no part of it needs to start at zero (each
 * kernel writes what a later one reads); calls that overlap on one GPU -- on different streams
 * or threads -- race on it. */
int dllm_layer_sparse_noalloc(const dllm_model *model, int32_t layer, void *x_act, const int32_t *idx,
                              const int32_t *n_active, int32_t k_max, void *k_cache, void *v_cache, void *stream);

/* Fused confidence / argmax / local-KL pass over the vocabulary ([SL] 2.1
 * item 1: D = KL(p_t || p_{t-1}); [ES] Eq. 1 confidence c).
 *  logits: device [R, V] fp32; row_pos: device [R], row r belongs to flat
 *  position row_pos[r] = b*S + i, or -1 (dead row, skipped).
 *  logits_prev: device [B*S, V] of prev_dtype (DLLM_F32 or DLLM_BF16) or NULL.
 *  When non-NULL the row's previous logits are read (if have_prev) and then
 *  overwritten with logits[r] (rounded to bf16 for a bf16 state, where the
 *  KL compares the bf16-rounded current logits with the stored ones).
 *  conf, argmax: device [B*S]; kl: device [B*S] or NULL (+inf without have_prev).
 *  exclude_id: vocabulary id treated as -inf (the mask token), or -1. */
int dllm_confidence_kl(const float *logits, void *logits_prev, int32_t prev_dtype, const int32_t *row_pos, int32_t R,
                       int32_t V, int32_t exclude_id, int32_t have_prev, float *conf,
                       int32_t *argmax, float *kl, void *stream);

/* The plan of the packed-weight product over M active rows (host only; no device call):
 * returns 1 and stores the waves per workgroup (*nw, one 32-column block each) and the K splits
 * (*splits, fp32 partials) when the packed path takes an M x N x K product ([ES] 2.1 item 2:
 * the active rows' products at batch 1 stream the weights), else returns 0.  swiglu != 0 asks
 * for the fused gate/up product (N = 2F packed columns, never split).  nw/splits may be NULL. */
int dllm_packed_plan(int32_t M, int32_t N, int32_t K, int32_t swiglu, int32_t *nw, int32_t *splits);

/* Repacks a bf16 weight W [N, K] (nn.Linear layout) into MFMA B-fragment order for the
 * active-row products ([ES] 2.1 item 2: at batch 1 they stream the weights): fragment
 * (nb, ks) -- 32 output columns x 16 reduction elements -- is 1 KB at element
 * ((ks / 4) * (N / 32) + nb) * 2048 + (ks % 4) * 512 (stage-major: the 64-element stages of all
 * column blocks one after the other), lane l element e holding
 * W[row(32 nb + l % 32)][16 ks + 8 (l / 32) + e].
 * With interleave_f = F > 0, W is the stacked [gate; up] [2F, K] and packed row 32 nb + r is
 * gate row 16 nb + r (r < 16) or up row F + 16 nb + r - 16, so each output's two factors meet
 * in one accumulator.
 *  w: device [N, K] bf16; w_packed: device, N*K bf16 elements, caller-owned, not aliasing w.
 *  N % 32 == 0, K % 64 == 0; interleave_f is 0 or N / 2 (then a multiple of 16). */
int dllm_pack_weight(const void *w, void *w_packed, int32_t N, int32_t K, int32_t interleave_f, void *stream);

/* Device planner of one dilated unmasking round ([DUS] technical summary
 * section 2: a block of `block` positions is decoded in R = ceil(log_a block)
 * rounds, round r taking the offsets that are multiples of a^(R-1-r) and were
 * not taken by an earlier, coarser round).  For every sequence b and every
 * offset o of round `round` of the block [lo, lo + block):
 *     force[b*S + lo + o] = max(force[b*S + lo + o], mark).
 * Other positions are untouched.  With mark = 1 the round's positions join the
 * active set of the next dllm_skip_step (whatever their score) and are the ones
 * DLLM_UNMASK_FORCED unmasks; a locked position (2) stays locked.
 *  force: device [B, S] u8.  rounds: R, or 0 for ceil(log_a block) (1 for a
 *  single position).  a >= 2, 0 <= round < R, 1 <= mark <= 255,
 *  0 <= lo, lo + block <= S.  Invalid arguments return DLLM_EINVAL/ESHAPE
 *  before any launch. */
int dllm_dus_mark(uint8_t *force, int32_t B, int32_t S, int32_t lo, int32_t block, int32_t a,
                  int32_t rounds, int32_t round, int32_t mark, void *stream);

/* One full denoising iteration ([ES] 2.1; [SL] 2.1): embed, dense layers
 * below the boundary, score + select at the boundary, sparse layers,
 * final-hidden scatter, LM head on the active rows, confidence/KL, then the
 * SureLock lock update and/or confidence unmasking of [block_lo, block_hi).
 * On a full step every row is active, whatever state->k_max is. */
int dllm_skip_step(const dllm_model *model, dllm_state *state, const dllm_step_cfg *cfg, void *stream);

/* Achievable-peak probes for measurement (nothing on the denoising path uses them): the measured
 * denominators beside the datasheet peaks.
 *  DLLM_PROBE_COPY: copies the first half of buf into the second half, iters times (a plain HBM
 *    stream, four 16-byte loads in flight per thread); *work = bytes read + written.
 *  DLLM_PROBE_MFMA: a loop of iters steps of four independent v_mfma_f32_32x32x16_bf16 chains per
 *    wave on register operands, 2048 workgroups of 4 waves (8 per CU); buf must hold at least
 *    2048 * 256 floats (written only in a case the sums cannot reach); *work = flops.
 *  DLLM_PROBE_READ: a nontemporal read of buf past its first 512 KiB, iters times (the way the
 *    products stream their weights); the first 512 KiB take one word per thread, written only in a
 *    case the folded words cannot be known to avoid; bytes must exceed 1 MiB; *work = bytes read.
 *  The work is enqueued on `stream`; the caller times it (e.g. with events). Errors: DLLM_EINVAL
 *  (null pointers, unaligned buf, iters < 1, unknown kind), DLLM_ESHAPE (buf too small). */
enum { DLLM_PROBE_COPY = 0, DLLM_PROBE_MFMA = 1, DLLM_PROBE_READ = 2 };
int dllm_peak_probe(int32_t kind, void *buf, size_t bytes, int32_t iters, double *work, void *stream);

/* Precondition bits recorded by the checking build. */
enum {
  DLLM_CHECK_ACTIVE_COUNT = 1, /* n_active[b] outside [0, k_max] */
  DLLM_CHECK_INDEX_RANGE = 2,  /* a live idx entry outside [0, S) (the row is skipped) */
  DLLM_CHECK_INDEX_ORDER = 4,  /* live idx entries of a sequence not strictly ascending */
  DLLM_CHECK_TOKEN_RANGE = 8   /* a token id outside [0, V) (it is clamped) */
};

/* Debug aid.  libdllm_check.so is the same library built with -DDLLM_CHECK: the kernels that
 * consume caller-supplied indices (dllm_layer_sparse and its allocation-free variant, the gather /
 * scatter entry points) and token ids (dllm_skip_step) verify them on the device and OR the
 * DLLM_CHECK_* bits of any violation into a per-GPU error word, while keeping every access in
 * bounds.  dllm_check_word synchronises the current device, stores the word in *word and, with
 * clear != 0, resets it.  In the normal build nothing is checked: it stores 0 and returns
 * DLLM_EINVAL without touching the device. */
int dllm_check_word(uint32_t *word, int32_t clear);

/* Human-readable text of a dllm_status. */
const char *dllm_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int dllm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
