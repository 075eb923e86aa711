// C ABI of libdllm: argument validation, workspace planning and the launch
// order of one token-skipping denoising iteration.  Everything is enqueued on
// the caller's stream; nothing is allocated and no host synchronisation
// happens inside a call (the active-row count stays on the device; grids are
// sized for the row capacity and dead tiles exit early).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/dllm.h"
#include "common.h"
#include "kernels.h"

using namespace dllm;

// Library-owned scratch for callers that cannot allocate (code under graph capture, tight serving
// loops): one file-scope device array, which every GPU the library runs on holds until the process
// ends.  In host code `scratch` names a host-side stand-in, not a device address: the address of a
// device's copy comes from hipGetSymbolAddress with that device current, once per device, and only
// that address is handed to kernels (as the workspace pointer of an ordinary layer call).
static __device__ __align__(256) uint8_t scratch[DLLM_NOALLOC_SCRATCH_BYTES];

// Error word of the checking build (-DDLLM_CHECK): the precondition bits kernels set on this GPU.
static __device__ uint32_t check_word_dev;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int esize(int dtype) { return dtype == DLLM_F32 ? 4 : 2; }

#define DLLM_TRY(expr)                       \
  do {                                       \
    if ((expr) != hipSuccess) return DLLM_ELAUNCH; \
  } while (0)

// Measurement hook of one call (dllm_step_cfg.timing): brackets the launches of one kernel class
// with caller-created events on the call's stream.  `err` holds the status of the start record;
// stop() records the end and counts the pair only when both records succeeded.
struct TimedRegion {
  dllm_timing* t = nullptr;
  hipStream_t s;
  int slot = -1;
  hipError_t err = hipSuccess;
  TimedRegion(dllm_timing* g, int kernel, int rows, hipStream_t st) : s(st) {
    if (!g || g->kernel != kernel || (g->max_rows > 0 && rows > g->max_rows) || g->count >= g->capacity) return;
    t = g;
    slot = g->count;
    err = hipEventRecord((hipEvent_t)g->start[slot], s);
    if (err != hipSuccess) t = nullptr;
  }
  hipError_t stop() {
    if (!t) return err;
    err = hipEventRecord((hipEvent_t)t->stop[slot], s);
    if (err == hipSuccess) t->count = slot + 1;
    t = nullptr;
    return err;
  }
};

bool timing_ok(const dllm_timing* t) {
  return !t || (t->capacity >= 0 && t->count >= 0 && (t->capacity == 0 || (t->start && t->stop)));
}

// Workspace layout for (dims, dtype, k_max).
struct WsLayout {
  size_t xfull, xact, xn, q, o, h, part, attn, vpart, logits, scores, idx_id, nact_full, rowpos_d, rowpos_s,
      nforce, row_of, old_row, cand_idx, cand_n, cand_rp, total;
};

long max_part_floats(const dllm_dims& d, int dtype, long M) {
  const int NQKV = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  const int HQD = d.n_heads * d.head_dim;
  // QKV, O, gate/up, down, and the V projection alone (the per-layer cache's V feature)
  const int Ns[5] = {NQKV, d.d, 2 * d.d_ff, d.d, d.n_kv_heads * d.head_dim};
  const int Ks[5] = {d.d, HQD, d.d, d.d_ff, d.d};
  long best = 0;
  for (int i = 0; i < 5; ++i) {
    const GemmPlan p = gemm_plan(dtype, (int)M, Ns[i], Ks[i]);
    best = std::max(best, (long)p.splits * M * Ns[i]);
  }
  // the packed products (QKV, down) that write split-K partials
  if (dtype == DLLM_BF16) {
    for (int i : {0, 3}) {
      const PackedPlan pp = packed_plan((int)M, Ns[i], Ks[i], false);
      if (pp.ok) best = std::max(best, (long)pp.splits * M * Ns[i]);
    }
  }
  return best;
}

bool plan_ws(const dllm_dims& d, int dtype, int k_max, WsLayout& L) {
  const long Rd = (long)d.B * d.S, Rs = (long)d.B * k_max, R = std::max(Rd, Rs);
  const int es = esize(dtype);
  const long HQD = (long)d.n_heads * d.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L.xfull = take(Rd * d.d * es);
  L.xact = take(Rs * d.d * es);
  L.xn = take(R * d.d * es);
  L.q = take(R * HQD * es);
  L.o = take(R * HQD * es);
  L.h = take(R * (long)d.d_ff * es);
  L.part = take(std::max(max_part_floats(d, dtype, Rd), max_part_floats(d, dtype, Rs)) * sizeof(float));
  L.attn = take(std::max(attention_part_bytes(dtype, d.B, d.S, d.S, d.n_heads, d.n_kv_heads),
                         attention_part_bytes(dtype, d.B, d.S, k_max, d.n_heads, d.n_kv_heads)));
  L.vpart = take(std::max(conf_kl_part_bytes((int)Rd, d.vocab), conf_kl_part_bytes((int)Rs, d.vocab)));
  L.logits = take(R * (long)d.vocab * sizeof(float));
  L.scores = take(Rd * sizeof(float));
  L.idx_id = take(Rd * sizeof(int32_t));
  L.nact_full = take(d.B * sizeof(int32_t));
  L.rowpos_d = take(Rd * sizeof(int32_t));
  L.rowpos_s = take(Rs * sizeof(int32_t));
  L.nforce = take(Rd);                     // nested boundaries: candidate marks per position
  L.row_of = take(Rd * sizeof(int32_t));   //   active row of each position
  L.old_row = take(Rs * sizeof(int32_t));  //   row before narrowing of each row after it
  L.cand_idx = take(Rd * sizeof(int32_t)); // per-layer cache, V feature: unlocked positions,
  L.cand_n = take(d.B * sizeof(int32_t));  //   their count per sequence,
  L.cand_rp = take(Rd * sizeof(int32_t));  //   and their row positions
  L.total = off;
  return true;
}

// What one layer on B * k_max active rows needs (dllm_layer_sparse's kernels): the normalised
// rows, Q, the attention output, the SwiGLU rows, the split-K partials, split-KV partials and the
// row positions.  The other offsets stay 0 (unused by a layer call).
size_t plan_layer_ws(const dllm_dims& d, int dtype, int k_max, WsLayout& L) {
  L = WsLayout{};
  const long Rs = (long)d.B * k_max;
  const int es = esize(dtype);
  const long HQD = (long)d.n_heads * d.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L.xn = take(Rs * d.d * es);
  L.q = take(Rs * HQD * es);
  L.o = take(Rs * HQD * es);
  L.h = take(Rs * (long)d.d_ff * es);
  L.part = take(max_part_floats(d, dtype, Rs) * sizeof(float));
  L.attn = take(attention_part_bytes(dtype, d.B, d.S, k_max, d.n_heads, d.n_kv_heads));
  L.rowpos_s = take(Rs * sizeof(int32_t));
  L.total = off;
  return off;
}

int check_dims(const dllm_dims* d, int dtype) {
  if (!d) return DLLM_EINVAL;
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
  if (d->B < 1 || d->S < 1 || d->d < 1 || d->n_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->d_ff < 1 ||
      d->vocab < 2 || d->n_layers < 1)
    return DLLM_ESHAPE;
  if (d->n_heads % d->n_kv_heads) return DLLM_ESHAPE;
  if (d->head_dim % 2) return DLLM_ESHAPE;
  if (dtype == DLLM_BF16) {
    // MFMA GEMM: every reduction dim a multiple of 64; attention head dim 128
    if (d->head_dim != 128 || d->d % 64 || (d->n_heads * d->head_dim) % 64 || d->d_ff % 64) return DLLM_ESHAPE;
    // 32-bit buffer offsets: a GEMM tile (up to 256 activation rows, or the gate..up span of
    // the SwiGLU weight) and one sequence's K/V cache of a layer stay under 2 GiB
    long kmax = d->d;
    if ((long)d->n_heads * d->head_dim > kmax) kmax = (long)d->n_heads * d->head_dim;
    if (d->d_ff > kmax) kmax = d->d_ff;
    const long lim = 1L << 31;
    if (256L * kmax * 2 >= lim || ((long)d->d_ff + 128) * d->d * 2 >= lim ||
        (long)d->S * d->n_kv_heads * d->head_dim * 2 >= lim)
      return DLLM_ESHAPE;
  } else {
    if ((d->head_dim != 64 && d->head_dim != 128) || d->d % 4 || d->d_ff % 4) return DLLM_ESHAPE;
  }
  if ((long)d->B * d->S > (1L << 30)) return DLLM_ESHAPE;
  return DLLM_OK;
}

int check_width(int width, int dtype) {
  if (width < 1) return DLLM_ESHAPE;
  return (width % (dtype == DLLM_F32 ? 4 : 8)) ? DLLM_ESHAPE : DLLM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Ctx {
  const dllm_model* m;
  const dllm_dims* d;
  int dtype;
  char* ws;
  WsLayout L;
  hipStream_t s;
  dllm_timing* timing = nullptr;  // this call's measurement hook, or null
  template <typename T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(ws + off);
  }
};

// One layer on rows r = b*kx + j (live iff j < nact[b]); xn holds rmsnorm(x) * attn_norm on entry.
int run_layer(const Ctx& c, int l, void* x, const int32_t* nact, const int32_t* row_pos, int kx, void* kc, void* vc,
              const void* next_g, void* out_scatter = nullptr) {
  const dllm_dims& d = *c.d;
  const dllm_layer_w& w = c.m->layers[l];
  const int R = d.B * kx;
  const int HQD = d.n_heads * d.head_dim;
  const int NQKV = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  float* part = c.at<float>(c.L.part);
  void* xn = c.ws + c.L.xn;
  void* q = c.ws + c.L.q;
  void* o = c.ws + c.L.o;
  void* h = c.ws + c.L.h;
  const float eps = c.m->rms_eps;

  GemmPlan p = gemm_plan(c.dtype, R, NQKV, d.d);
  {
    const PackedPlan pp = (c.dtype == DLLM_BF16 && w.w_qkv_packed) ? packed_plan(R, NQKV, d.d, false) : PackedPlan{};
    TimedRegion t(c.timing, DLLM_TK_QKV, R, c.s);
    DLLM_TRY(t.err);
    if (pp.ok) {
      DLLM_TRY(launch_gemm_packed(pp, xn, w.w_qkv_packed, part, nullptr, R, NQKV, d.d, 0, nact, kx, c.s));
      p.splits = pp.splits;
    } else {
      DLLM_TRY(launch_gemm(c.dtype, p, xn, w.w_qkv, part, R, NQKV, d.d, nact, kx, c.s));
    }
    DLLM_TRY(t.stop());
  }
  DLLM_TRY(launch_qkv_epilogue(c.dtype, part, p.splits, (long)R * NQKV, row_pos, R, d.S, d.n_heads, d.n_kv_heads,
                               d.head_dim, c.m->rope_base, q, kc, vc, c.s));
  {
    TimedRegion t(c.timing, DLLM_TK_ATTN, R, c.s);
    DLLM_TRY(t.err);
    DLLM_TRY(launch_attention(c.dtype, q, kc, vc, o, nact, d.B, d.S, kx, d.n_heads, d.n_kv_heads, d.head_dim,
                              c.at<float>(c.L.attn), c.s));
    DLLM_TRY(t.stop());
  }
  p = gemm_plan(c.dtype, R, d.d, HQD);
  {
    TimedRegion t(c.timing, DLLM_TK_O, R, c.s);
    DLLM_TRY(t.err);
    DLLM_TRY(launch_gemm(c.dtype, p, o, w.w_o, part, R, d.d, HQD, nact, kx, c.s));
    DLLM_TRY(t.stop());
  }
  DLLM_TRY(launch_resid_norm(c.dtype, part, p.splits, (long)R * d.d, row_pos, R, d.d, x, w.ffn_norm, eps, xn, c.s));
  if (c.dtype == DLLM_BF16) {
    const PackedPlan pp = w.w_gate_up_packed ? packed_plan(R, 2 * d.d_ff, d.d, true) : PackedPlan{};
    p = gemm_plan(c.dtype, R, d.d_ff, d.d, true);
    TimedRegion t(c.timing, DLLM_TK_FFN_UP, R, c.s);
    DLLM_TRY(t.err);
    if (pp.ok)
      DLLM_TRY(launch_gemm_packed(pp, xn, w.w_gate_up_packed, nullptr, h, R, 2 * d.d_ff, d.d, d.d_ff, nact, kx, c.s));
    else
      DLLM_TRY(launch_gemm_swiglu(p, xn, w.w_gate_up, h, R, d.d_ff, d.d, nact, kx, c.s));
    DLLM_TRY(t.stop());
  } else {
    p = gemm_plan(c.dtype, R, 2 * d.d_ff, d.d);
    TimedRegion t(c.timing, DLLM_TK_FFN_UP, R, c.s);
    DLLM_TRY(t.err);
    DLLM_TRY(launch_gemm(c.dtype, p, xn, w.w_gate_up, part, R, 2 * d.d_ff, d.d, nact, kx, c.s));
    DLLM_TRY(launch_swiglu(c.dtype, part, p.splits, (long)R * 2 * d.d_ff, row_pos, R, d.d_ff, h, c.s));
    DLLM_TRY(t.stop());
  }
  p = gemm_plan(c.dtype, R, d.d, d.d_ff);
  {
    const PackedPlan pp = (c.dtype == DLLM_BF16 && w.w_down_packed) ? packed_plan(R, d.d, d.d_ff, false)
                                                                     : PackedPlan{};
    TimedRegion t(c.timing, DLLM_TK_FFN_DOWN, R, c.s);
    DLLM_TRY(t.err);
    if (pp.ok) {
      DLLM_TRY(launch_gemm_packed(pp, h, w.w_down_packed, part, nullptr, R, d.d, d.d_ff, 0, nact, kx, c.s));
      p.splits = pp.splits;
    } else {
      DLLM_TRY(launch_gemm(c.dtype, p, h, w.w_down, part, R, d.d, d.d_ff, nact, kx, c.s));
    }
    DLLM_TRY(t.stop());
  }
  DLLM_TRY(launch_resid_norm(c.dtype, part, p.splits, (long)R * d.d, row_pos, R, d.d, x, next_g, eps, xn, c.s,
                             out_scatter));
  return DLLM_OK;
}

int check_model(const dllm_model* m) {
  if (!m) return DLLM_EINVAL;
  int st = check_dims(&m->dims, m->dtype);
  if (st) return st;
  if (!m->embed || !m->layers || !m->final_norm || !m->lm_head) return DLLM_EINVAL;
  if (m->lm_head_packed && !aligned16(m->lm_head_packed)) return DLLM_EINVAL;  // 16-byte fragment loads
  if (m->mask_id < -1 || m->mask_id >= m->dims.vocab) return DLLM_EINVAL;
  if (!(m->rope_base > 0.f) || !(m->rms_eps >= 0.f)) return DLLM_EINVAL;
  for (int l = 0; l < m->dims.n_layers; ++l) {
    const dllm_layer_w& w = m->layers[l];
    if (!w.attn_norm || !w.w_qkv || !w.w_o || !w.ffn_norm || !w.w_gate_up || !w.w_down) return DLLM_EINVAL;
    for (const void* pk : {w.w_gate_up_packed, w.w_down_packed, w.w_qkv_packed})
      if (pk && !aligned16(pk)) return DLLM_EINVAL;
  }
  return DLLM_OK;
}

// ---- allocation-free layer calls ----
// The address of the scratch array's copy on one device is resolved once per device (below).
constexpr size_t kScratchBytes = DLLM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // the address of `scratch` on each device, once resolved

// This thread's current device's copy of `scratch` (resolved on its first use on that device).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DLLM_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DLLM_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DLLM_OK;
}

#ifdef DLLM_CHECK
void* g_check_ptr[kMaxDevices] = {};  // the address of the error word on each device, once resolved
#endif

// The current device's error word in the checking build (null in the normal build, where the
// kernels compile their checks out).
uint32_t* check_word() {
#ifdef DLLM_CHECK
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_check_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_word_dev)) != hipSuccess) return nullptr;
    g_check_ptr[dev] = p;
  }
  return (uint32_t*)g_check_ptr[dev];
#else
  return nullptr;
#endif
}

// dllm_layer_sparse on a workspace laid out by plan_layer_ws (or plan_ws).
int layer_call(const dllm_model* model, int32_t layer, void* x_act, const int32_t* idx, const int32_t* n_active,
               int32_t k_max, void* k_cache, void* v_cache, Ctx& c) {
  const dllm_dims& d = model->dims;
  int32_t* row_pos = c.at<int32_t>(c.L.rowpos_s);
  const int R = d.B * k_max;
  DLLM_TRY(launch_row_pos(idx, n_active, d.B, d.S, k_max, row_pos, c.s, check_word()));
  // xn = rmsnorm(x_act) * attn_norm (scatter mode with no copy target = norm only)
  DLLM_TRY(launch_scatter_norm(c.dtype, x_act, row_pos, R, d.d, nullptr, model->layers[layer].attn_norm,
                               model->rms_eps, c.ws + c.L.xn, c.s));
  return run_layer(c, layer, x_act, n_active, row_pos, k_max, k_cache, v_cache, nullptr);
}

int check_layer_args(const dllm_model* model, int32_t layer, const void* x_act, const int32_t* idx,
                     const int32_t* n_active, int32_t k_max, const void* k_cache, const void* v_cache) {
  int st = check_model(model);
  if (st) return st;
  const dllm_dims& d = model->dims;
  if (layer < 0 || layer >= d.n_layers) return DLLM_EINVAL;
  if (!x_act || !idx || !n_active || !k_cache || !v_cache) return DLLM_EINVAL;
  if (k_max < 1 || k_max > d.S) return DLLM_ESHAPE;
  if (!aligned16(x_act)) return DLLM_EINVAL;
  return DLLM_OK;
}

}  // namespace

extern "C" {

int dllm_version(void) { return 300; }

int dllm_peak_probe(int32_t kind, void* buf, size_t bytes, int32_t iters, double* work, void* stream) {
  if (!buf || !work || iters < 1) return DLLM_EINVAL;
  if (!aligned16(buf)) return DLLM_EINVAL;
  if (kind == DLLM_PROBE_COPY) {
    if (bytes < 32) return DLLM_ESHAPE;
  } else if (kind == DLLM_PROBE_MFMA) {
    if (bytes < (size_t)2048 * 256 * sizeof(float)) return DLLM_ESHAPE;
  } else if (kind == DLLM_PROBE_READ) {
    if (bytes <= ((size_t)1 << 20)) return DLLM_ESHAPE;
  } else {
    return DLLM_EINVAL;
  }
  DLLM_TRY(launch_peak_probe(kind, buf, bytes, iters, work, (hipStream_t)stream));
  return DLLM_OK;
}

int dllm_check_word(uint32_t* word, int32_t clear) {
  if (!word) return DLLM_EINVAL;
  *word = 0;
#ifdef DLLM_CHECK
  uint32_t* p = check_word();
  if (!p) return DLLM_ELAUNCH;
  if (hipDeviceSynchronize() != hipSuccess) return DLLM_ELAUNCH;
  if (hipMemcpy(word, p, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return DLLM_ELAUNCH;
  if (clear) {
    const uint32_t zero = 0;
    if (hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess) return DLLM_ELAUNCH;
  }
  return DLLM_OK;
#else
  (void)clear;
  return DLLM_EINVAL;  // not a checking build: nothing is recorded
#endif
}

const char* dllm_status_string(int status) {
  switch (status) {
    case DLLM_OK: return "ok";
    case DLLM_EINVAL: return "invalid argument";
    case DLLM_ESHAPE: return "unsupported or inconsistent shape";
    case DLLM_EDTYPE: return "unknown dtype";
    case DLLM_EWORKSPACE: return "workspace missing or too small";
    case DLLM_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t dllm_workspace_size(const dllm_dims* dims, int32_t dtype, int32_t k_max) {
  if (check_dims(dims, dtype) != DLLM_OK || k_max < 1 || k_max > dims->S) return 0;
  WsLayout L;
  plan_ws(*dims, dtype, k_max, L);
  return L.total;
}

int dllm_score_select(const void* h_cur, const void* h_prev, void* h_next, int32_t dtype, const float* conf_prev,
                      const float* kl_prev, const uint8_t* force, int32_t B, int32_t S, int32_t width,
                      const dllm_score_cfg* cfg, float* score_out, int32_t* idx_out, int32_t* n_active_out,
                      int32_t k_max, void* stream) {
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
  if (!cfg || !h_cur || !h_prev || !conf_prev || !score_out || !idx_out || !n_active_out) return DLLM_EINVAL;
  if (B < 1 || S < 1 || k_max < 1 || k_max > S) return DLLM_ESHAPE;
  if (check_width(width, dtype)) return DLLM_ESHAPE;
  if (!aligned16(h_cur) || !aligned16(h_prev) || (h_next && !aligned16(h_next))) return DLLM_EINVAL;
  if (cfg->var < DLLM_VAR_L1N || cfg->var > DLLM_VAR_NONE) return DLLM_EINVAL;
  if (cfg->var == DLLM_VAR_KL && !kl_prev) return DLLM_EINVAL;
  if (cfg->sel < DLLM_SEL_TOPK || cfg->sel > DLLM_SEL_UNLOCKED) return DLLM_EINVAL;
  if (cfg->sel != DLLM_SEL_UNLOCKED && (cfg->k < 0 || cfg->k > k_max)) return DLLM_EINVAL;
  if (cfg->sel == DLLM_SEL_UNLOCKED && k_max != S) return DLLM_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  DLLM_TRY(launch_score(dtype, h_cur, h_prev, h_next, conf_prev, kl_prev, force, B * S, width, cfg->alpha,
                        cfg->conf_inverted, cfg->var, score_out, s));
  DLLM_TRY(launch_select(score_out, force, B, S, cfg->sel, cfg->k, cfg->tau, k_max, idx_out, n_active_out, s));
  return DLLM_OK;
}

static int gather_scatter(bool gather, const void* src, const int32_t* idx, const int32_t* n_active, int32_t B,
                          int32_t S, int32_t k_max, int32_t width, int32_t dtype, void* dst, void* stream,
                          int32_t* row_pos_ws) {
  (void)row_pos_ws;
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return DLLM_EDTYPE;
  if (!src || !idx || !n_active || !dst) return DLLM_EINVAL;
  if (B < 1 || S < 1 || k_max < 1 || k_max > S || check_width(width, dtype)) return DLLM_ESHAPE;
  if (!aligned16(src) || !aligned16(dst)) return DLLM_EINVAL;
  return DLLM_OK;
}

// Gather/scatter compute the row positions on the fly from idx/n_active (no workspace).
namespace {
__global__ void k_gs_rows(bool gather, const uint4* __restrict__ src, const int32_t* __restrict__ idx,
                          const int32_t* __restrict__ n_active, int S, int k_max, int nchunk, uint4* __restrict__ dst,
                          uint32_t* chk) {
  const int r = blockIdx.x;
  const int b = r / k_max, j = r - b * k_max;
  const int na = n_active[b];
  if (j == 0 && threadIdx.x == 0 && (na < 0 || na > k_max)) check_flag(chk, kChkActiveCount);
  if (j >= na) return;
  const int i = idx[r];
  if (i < 0 || i >= S) {
    if (threadIdx.x == 0) check_flag(chk, kChkIndexRange);
    return;
  }
  if (j > 0 && threadIdx.x == 0 && idx[r - 1] >= i) check_flag(chk, kChkIndexOrder);
  const long pos = (long)b * S + i;
  const uint4* s4 = src + (gather ? pos : (long)r) * nchunk;
  uint4* d4 = dst + (gather ? (long)r : pos) * nchunk;
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) d4[c] = s4[c];
}
}  // namespace

int dllm_gather_rows(const void* src, const int32_t* idx, const int32_t* n_active, int32_t B, int32_t S,
                     int32_t k_max, int32_t width, int32_t dtype, void* dst, void* stream) {
  int st = gather_scatter(true, src, idx, n_active, B, S, k_max, width, dtype, dst, stream, nullptr);
  if (st) return st;
  const int nchunk = width * esize(dtype) / 16;
  hipLaunchKernelGGL(k_gs_rows, dim3(B * k_max), dim3(256), 0, (hipStream_t)stream, true, (const uint4*)src, idx,
                     n_active, S, k_max, nchunk, (uint4*)dst, check_word());
  return hipGetLastError() == hipSuccess ? DLLM_OK : DLLM_ELAUNCH;
}

int dllm_scatter_rows(const void* src, const int32_t* idx, const int32_t* n_active, int32_t B, int32_t S,
                      int32_t k_max, int32_t width, int32_t dtype, void* dst, void* stream) {
  int st = gather_scatter(false, src, idx, n_active, B, S, k_max, width, dtype, dst, stream, nullptr);
  if (st) return st;
  const int nchunk = width * esize(dtype) / 16;
  hipLaunchKernelGGL(k_gs_rows, dim3(B * k_max), dim3(256), 0, (hipStream_t)stream, false, (const uint4*)src, idx,
                     n_active, S, k_max, nchunk, (uint4*)dst, check_word());
  return hipGetLastError() == hipSuccess ? DLLM_OK : DLLM_ELAUNCH;
}

int dllm_layer_sparse(const dllm_model* model, int32_t layer, void* x_act, const int32_t* idx,
                      const int32_t* n_active, int32_t k_max, void* k_cache, void* v_cache, void* ws, size_t ws_bytes,
                      void* stream) {
  const int st = check_layer_args(model, layer, x_act, idx, n_active, k_max, k_cache, v_cache);
  if (st) return st;
  Ctx c{model, &model->dims, model->dtype, (char*)ws, {}, (hipStream_t)stream};
  plan_ws(model->dims, c.dtype, k_max, c.L);
  if (!ws || ws_bytes < c.L.total) return DLLM_EWORKSPACE;
  return layer_call(model, layer, x_act, idx, n_active, k_max, k_cache, v_cache, c);
}

int dllm_layer_sparse_noalloc(const dllm_model* model, int32_t layer, void* x_act, const int32_t* idx,
                              const int32_t* n_active, int32_t k_max, void* k_cache, void* v_cache, void* stream) {
  const int st = check_layer_args(model, layer, x_act, idx, n_active, k_max, k_cache, v_cache);
  if (st) return st;
  Ctx c{model, &model->dims, model->dtype, nullptr, {}, (hipStream_t)stream};
  if (plan_layer_ws(model->dims, c.dtype, k_max, c.L) > kScratchBytes) return DLLM_EWORKSPACE;
  void* base = nullptr;
  const int sr = current_scratch(&base);
  if (sr) return sr;
  c.ws = (char*)base;
  return layer_call(model, layer, x_act, idx, n_active, k_max, k_cache, v_cache, c);
}

int dllm_confidence_kl(const float* logits, void* logits_prev, int32_t prev_dtype, const int32_t* row_pos, int32_t R,
                       int32_t V, int32_t exclude_id, int32_t have_prev, float* conf, int32_t* argmax, float* kl,
                       void* stream) {
  if (!logits || !row_pos || !conf || !argmax) return DLLM_EINVAL;
  if (prev_dtype != DLLM_F32 && prev_dtype != DLLM_BF16) return DLLM_EDTYPE;
  if (R < 0 || V < 2 || exclude_id >= V) return DLLM_ESHAPE;
  DLLM_TRY(launch_conf_kl(logits, logits_prev, prev_dtype, row_pos, R, V, exclude_id, have_prev, conf, argmax, kl,
                          nullptr, (hipStream_t)stream));
  return DLLM_OK;
}

int dllm_packed_plan(int32_t M, int32_t N, int32_t K, int32_t swiglu, int32_t* nw, int32_t* splits) {
  const PackedPlan p = packed_plan(M, N, K, swiglu != 0);
  if (nw) *nw = p.ok ? p.nw : 0;
  if (splits) *splits = p.ok ? p.splits : 0;
  return p.ok ? 1 : 0;
}

int dllm_pack_weight(const void* w, void* w_packed, int32_t N, int32_t K, int32_t interleave_f, void* stream) {
  if (!w || !w_packed || w == w_packed) return DLLM_EINVAL;
  if (!aligned16(w) || !aligned16(w_packed)) return DLLM_EINVAL;
  if (N < 32 || K < 64 || N % 32 || K % 64) return DLLM_ESHAPE;
  if (interleave_f != 0 && (2L * interleave_f != N || interleave_f % 16)) return DLLM_ESHAPE;
  DLLM_TRY(launch_pack_frag(w, w_packed, N, K, interleave_f, (hipStream_t)stream));
  return DLLM_OK;
}

int dllm_dus_mark(uint8_t* force, int32_t B, int32_t S, int32_t lo, int32_t block, int32_t a, int32_t rounds,
                  int32_t round, int32_t mark, void* stream) {
  if (!force) return DLLM_EINVAL;
  if (B < 1 || S < 1 || block < 1 || lo < 0 || (long)lo + block > S) return DLLM_ESHAPE;
  if (a < 2 || rounds < 0 || mark < 1 || mark > 255) return DLLM_EINVAL;
  // R = ceil(log_a block) rounds by default (one round for a single position)
  int R = rounds;
  if (R == 0) {
    long p = 1;
    while (p < block) {
      p *= a;
      ++R;
    }
    if (R == 0) R = 1;
  }
  if (round < 0 || round >= R) return DLLM_EINVAL;
  // a^(R-1-round) and a^(R-round), clamped to the block length (no overflow for large R)
  auto clamped_pow = [&](int e) -> int {
    long p = 1;
    for (int i = 0; i < e && p < block; ++i) p *= a;
    return (int)(p < block ? p : block);
  };
  const int stride = clamped_pow(R - 1 - round);
  const int stride_prev = round == 0 ? 0 : clamped_pow(R - round);
  DLLM_TRY(launch_dus_mark(force, B, S, lo, block, stride, stride_prev, (uint8_t)mark, (hipStream_t)stream));
  return DLLM_OK;
}

int dllm_skip_step(const dllm_model* model, dllm_state* state, const dllm_step_cfg* cfg, void* stream) {
  int st = check_model(model);
  if (st) return st;
  if (!state || !cfg) return DLLM_EINVAL;
  if (state->logits_prev_dtype != DLLM_F32 && state->logits_prev_dtype != DLLM_BF16) return DLLM_EDTYPE;
  const dllm_dims& d = model->dims;
  const int L = d.n_layers, B = d.B, S = d.S;
  const int full = cfg->full_step ? 1 : 0;
  const int b_lay = cfg->boundary_layer;
  if (b_lay < 0 || b_lay > L) return DLLM_EINVAL;
  if (!state->tokens || !state->k_cache || !state->v_cache || !state->h_bnd[0] || !state->h_bnd[1] ||
      !state->h_fin || !state->conf || !state->kl || !state->argmax || !state->idx || !state->n_active)
    return DLLM_EINVAL;
  for (int l = 0; l < L; ++l)
    if (!state->k_cache[l] || !state->v_cache[l]) return DLLM_EINVAL;
  const int kx = state->k_max;
  if (kx < 1 || kx > S) return DLLM_ESHAPE;
  if (state->bnd_cur != 0 && state->bnd_cur != 1) return DLLM_EINVAL;
  const dllm_score_cfg& sc = cfg->score;
  if (!full) {
    if (!state->have_prev) return DLLM_EINVAL;  // a sparse step needs the previous boundary state
    if (sc.var < DLLM_VAR_L1N || sc.var > DLLM_VAR_NONE) return DLLM_EINVAL;
    if (sc.sel < DLLM_SEL_TOPK || sc.sel > DLLM_SEL_UNLOCKED) return DLLM_EINVAL;
    if (sc.sel != DLLM_SEL_UNLOCKED && (sc.k < 0 || sc.k > kx)) return DLLM_EINVAL;
    if (sc.sel == DLLM_SEL_UNLOCKED && kx != S) return DLLM_EINVAL;
  }
  if (cfg->unmask_n < 0 || cfg->unmask_n > 256) return DLLM_EINVAL;
  if (cfg->unmask_mode != DLLM_UNMASK_CONF && cfg->unmask_mode != DLLM_UNMASK_FORCED) return DLLM_EINVAL;
  if (cfg->unmask_n > 0 && cfg->unmask_mode == DLLM_UNMASK_FORCED && !state->force) return DLLM_EINVAL;
  if (cfg->unmask_n > 0 && (cfg->block_lo < 0 || cfg->block_hi > S || cfg->block_lo > cfg->block_hi))
    return DLLM_EINVAL;
  if (cfg->lock_kl_eps >= 0.f && !state->force) return DLLM_EINVAL;
  const int n_nested = cfg->n_nested;
  if (n_nested < 0 || n_nested > DLLM_MAX_NESTED) return DLLM_EINVAL;
  for (int j = 0, prev = b_lay; j < n_nested; prev = cfg->nested_layer[j], ++j) {
    if (cfg->nested_layer[j] <= prev || cfg->nested_layer[j] >= L) return DLLM_EINVAL;
    if (cfg->nested_k[j] < 0 || cfg->nested_k[j] > kx) return DLLM_EINVAL;
    if (!state->h_nested[j] || !aligned16(state->h_nested[j])) return DLLM_EINVAL;
  }
  if (cfg->layer_cache < 0 || cfg->layer_cache > DLLM_LCACHE_VALUE) return DLLM_EINVAL;
  const bool lcache = cfg->layer_cache != 0;
  const bool vfeat = cfg->layer_cache == DLLM_LCACHE_VALUE;
  if (lcache) {
    if (n_nested != 0 || b_lay >= L || !state->x_in_cache || !state->x_out_cache) return DLLM_EINVAL;
    for (int l = b_lay; l < L; ++l)
      if (!state->x_in_cache[l] || !state->x_out_cache[l] || !aligned16(state->x_in_cache[l]) ||
          !aligned16(state->x_out_cache[l]))
        return DLLM_EINVAL;
  }

  if (!timing_ok(cfg->timing)) return DLLM_EINVAL;

  Ctx c{model, &d, model->dtype, (char*)cfg->ws, {}, (hipStream_t)stream, cfg->timing};
  plan_ws(d, c.dtype, kx, c.L);
  if (!cfg->ws || cfg->ws_bytes < c.L.total) return DLLM_EWORKSPACE;
  const int es = esize(c.dtype);
  const size_t row_bytes = (size_t)d.d * es;
  const int Rd = B * S, Rs = B * kx;
  void* xfull = c.ws + c.L.xfull;
  void* xact = c.ws + c.L.xact;
  void* xn = c.ws + c.L.xn;
  int32_t* idx_id = c.at<int32_t>(c.L.idx_id);
  int32_t* nact_full = c.at<int32_t>(c.L.nact_full);
  int32_t* rp_d = c.at<int32_t>(c.L.rowpos_d);
  int32_t* rp_s = c.at<int32_t>(c.L.rowpos_s);
  void* h_prev = state->h_bnd[state->bnd_cur];
  void* h_next = state->h_bnd[1 - state->bnd_cur];
  const float eps = model->rms_eps;

  DLLM_TRY(launch_identity_rows(B, S, idx_id, nact_full, c.s, rp_d));  // every row, and its row position
  // embedding (+ first layer's norm when layer 0 runs dense)
  const bool l0_dense = full || b_lay > 0;
  DLLM_TRY(launch_embed_norm(c.dtype, model->embed, state->tokens, d.vocab, Rd, d.d,
                             l0_dense ? model->layers[0].attn_norm : nullptr, eps, xfull, xn, c.s, check_word()));

  auto boundary = [&]() -> int {
    if (full) {
      DLLM_TRY(launch_copy(xfull, h_next, (size_t)Rd * row_bytes, c.s));
      return DLLM_OK;
    }
    float* scores = c.at<float>(c.L.scores);
    {
      TimedRegion t(c.timing, DLLM_TK_SCORE, Rd, c.s);
      DLLM_TRY(t.err);
      DLLM_TRY(launch_score(c.dtype, xfull, h_prev, h_next, state->conf, state->kl, state->force, Rd, d.d, sc.alpha,
                            sc.conf_inverted, sc.var, scores, c.s));
      DLLM_TRY(t.stop());
    }
    {
      TimedRegion t(c.timing, DLLM_TK_SELECT, Rd, c.s);
      DLLM_TRY(t.err);
      DLLM_TRY(launch_select(scores, state->force, B, S, sc.sel, sc.k, sc.tau, kx, state->idx, state->n_active, c.s,
                             rp_s));
      DLLM_TRY(t.stop());
    }
    const void* g = (b_lay < L) ? model->layers[b_lay].attn_norm : model->final_norm;
    DLLM_TRY(launch_gather_norm(c.dtype, xfull, rp_s, Rs, d.d, xact, g, eps, xn, c.s));
    return DLLM_OK;
  };

  // nested boundary j at layer nl: re-score the active rows against the layer's cache, keep the
  // top nested_k[j], refresh the cache for every row that got here, compact the survivors
  auto nested = [&](int j, int nl) -> int {
    void* hc = state->h_nested[j];
    if (full) {
      DLLM_TRY(launch_copy(xfull, hc, (size_t)Rd * row_bytes, c.s));
      return DLLM_OK;
    }
    float* scores = c.at<float>(c.L.scores);
    uint8_t* nforce = c.at<uint8_t>(c.L.nforce);
    int32_t* row_of = c.at<int32_t>(c.L.row_of);
    int32_t* old_row = c.at<int32_t>(c.L.old_row);
    DLLM_TRY(launch_score_rows(c.dtype, xact, rp_s, Rs, hc, state->conf, state->kl, state->force, (long)Rd, d.d,
                               sc.alpha, sc.conf_inverted, sc.var, scores, nforce, row_of, c.s));
    DLLM_TRY(launch_select(scores, nforce, B, S, DLLM_SEL_TOPK, cfg->nested_k[j], 0.f, kx, state->idx,
                           state->n_active, c.s));
    DLLM_TRY(launch_scatter_norm(c.dtype, xact, rp_s, Rs, d.d, hc, nullptr, eps, nullptr, c.s));
    DLLM_TRY(launch_copy(xact, xfull, (size_t)Rs * row_bytes, c.s));  // xfull is idle past the boundary
    DLLM_TRY(launch_row_pos(state->idx, state->n_active, B, S, kx, rp_s, c.s));
    DLLM_TRY(launch_compose_rows(rp_s, row_of, Rs, old_row, c.s));
    DLLM_TRY(launch_gather_norm(c.dtype, xfull, old_row, Rs, d.d, xact, model->layers[nl].attn_norm, eps, xn, c.s));
    return DLLM_OK;
  };
  auto nested_at = [&](int l) -> int {
    for (int j = 0; j < n_nested; ++j)
      if (cfg->nested_layer[j] == l) return j;
    return -1;
  };

  // per-layer cache at layer l >= b: score every position against the layer's input cache,
  // compute the top k through the layer (refreshing both caches for them), every other position
  // takes its cached output; a full step computes every row and fills both caches
  // input rows of the next cached layer: the boundary's input, then each sparse layer's
  // output cache, which holds the current output of every row (no copy back into xfull)
  const void* xin = xfull;
  bool cand_ready = false;
  auto cached_layer = [&](int l) -> int {
    void* ci = state->x_in_cache[l];
    void* co = state->x_out_cache[l];
    const void* next_g = (l + 1 == L) ? model->final_norm : (full ? model->layers[l + 1].attn_norm : nullptr);
    if (full) {
      DLLM_TRY(launch_copy(xfull, ci, (size_t)Rd * row_bytes, c.s));
      const int r = run_layer(c, l, xfull, nact_full, rp_d, S, state->k_cache[l], state->v_cache[l], next_g);
      if (r) return r;
      DLLM_TRY(launch_copy(xfull, co, (size_t)Rd * row_bytes, c.s));
      return DLLM_OK;
    }
    float* scores = c.at<float>(c.L.scores);
    if (vfeat) {
      // the unlocked positions (the same for every layer of the step), in ascending order
      int32_t* cand_idx = c.at<int32_t>(c.L.cand_idx);
      int32_t* cand_n = c.at<int32_t>(c.L.cand_n);
      int32_t* cand_rp = c.at<int32_t>(c.L.cand_rp);
      if (!cand_ready) {
        DLLM_TRY(launch_select(scores, state->force, B, S, DLLM_SEL_UNLOCKED, S, 0.f, S, cand_idx, cand_n, c.s,
                               cand_rp));
        cand_ready = true;
      }
      // the layer's V projection of every candidate's current input (rows b*S + j, j < cand_n[b]),
      // stored in the element type, against the V the position holds in the layer's cache
      const int HKD = d.n_kv_heads * d.head_dim;
      const char* w_v = (const char*)model->layers[l].w_qkv + (size_t)(d.n_heads + d.n_kv_heads) * d.head_dim * d.d * es;
      float* part = c.at<float>(c.L.part);
      void* vnew = c.ws + c.L.q;  // idle until the layer runs
      DLLM_TRY(launch_gather_norm(c.dtype, xin, cand_rp, Rd, d.d, nullptr, model->layers[l].attn_norm, eps, xn, c.s));
      const GemmPlan pv = gemm_plan(c.dtype, Rd, HKD, d.d);
      DLLM_TRY(launch_gemm(c.dtype, pv, xn, w_v, part, Rd, HKD, d.d, cand_n, S, c.s));
      DLLM_TRY(launch_sum_store(c.dtype, part, pv.splits, (long)Rd * HKD, cand_rp, Rd, HKD, vnew, c.s));
      uint8_t* nforce = c.at<uint8_t>(c.L.nforce);
      DLLM_TRY(launch_score_rows(c.dtype, vnew, cand_rp, Rd, state->v_cache[l], state->conf, state->kl, state->force,
                                 (long)Rd, HKD, sc.alpha, sc.conf_inverted, sc.var, scores, nforce,
                                 c.at<int32_t>(c.L.row_of), c.s));
      DLLM_TRY(launch_select(scores, nforce, B, S, sc.sel, sc.k, sc.tau, kx, state->idx, state->n_active, c.s, rp_s));
    } else {
      DLLM_TRY(launch_score(c.dtype, xin, ci, nullptr, state->conf, state->kl, state->force, Rd, d.d, sc.alpha,
                            sc.conf_inverted, sc.var, scores, c.s));
      DLLM_TRY(launch_select(scores, state->force, B, S, sc.sel, sc.k, sc.tau, kx, state->idx, state->n_active, c.s,
                             rp_s));
    }
    // the selected rows, normalised for the layer, and their inputs recorded in the input cache
    DLLM_TRY(launch_gather_norm(c.dtype, xin, rp_s, Rs, d.d, xact, model->layers[l].attn_norm, eps, xn, c.s, ci));
    // the layer's outputs go to the output cache from its last residual kernel
    const int r = run_layer(c, l, xact, state->n_active, rp_s, kx, state->k_cache[l], state->v_cache[l], next_g, co);
    if (r) return r;
    xin = co;
    return DLLM_OK;
  };

  for (int l = 0; l < L; ++l) {
    if (lcache && l >= b_lay) {
      st = cached_layer(l);
      if (st) return st;
      continue;
    }
    if (l == b_lay) {
      st = boundary();
      if (st) return st;
    }
    const int jn = nested_at(l);
    if (jn >= 0) {
      st = nested(jn, l);
      if (st) return st;
    }
    const bool dense = full || l < b_lay;
    const void* next_g;
    if (l + 1 == L) next_g = model->final_norm;
    else if (!full && (l + 1 == b_lay || nested_at(l + 1) >= 0))
      next_g = nullptr;  // the boundary (or nested, or per-layer cache) gather normalises the active rows
    else next_g = model->layers[l + 1].attn_norm;
    if (dense)
      st = run_layer(c, l, xfull, nact_full, rp_d, S, state->k_cache[l], state->v_cache[l], next_g);
    else  // the last layer's residual kernel also writes the final hidden state of its rows
      st = run_layer(c, l, xact, state->n_active, rp_s, kx, state->k_cache[l], state->v_cache[l], next_g,
                     l + 1 == L ? state->h_fin : nullptr);
    if (st) return st;
  }
  if (b_lay == L) {
    st = boundary();
    if (st) return st;
  }

  // final hidden state of the computed rows; xn already holds rmsnorm(x) * final_norm
  const int R = full ? Rd : Rs;
  const int32_t* rp = full ? rp_d : rp_s;
  const int32_t* nact = full ? nact_full : state->n_active;
  const int kk = full ? S : kx;
  if (full) DLLM_TRY(launch_copy(xfull, state->h_fin, (size_t)Rd * row_bytes, c.s));
  else if (lcache || b_lay == L)  // otherwise the last sparse layer wrote them
    DLLM_TRY(launch_scatter_norm(c.dtype, xact, rp_s, Rs, d.d, state->h_fin, nullptr, eps, nullptr, c.s));

  float* logits = c.at<float>(c.L.logits);
  GemmPlan p = gemm_plan(c.dtype, R, d.vocab, d.d);
  p.splits = 1;
  const PackedPlan pp =
      (c.dtype == DLLM_BF16 && model->lm_head_packed) ? packed_plan_whole(R, d.vocab, d.d) : PackedPlan{};
  {
    TimedRegion t(c.timing, DLLM_TK_LM_HEAD, R, c.s);
    DLLM_TRY(t.err);
    if (pp.ok) DLLM_TRY(launch_gemm_packed(pp, xn, model->lm_head_packed, logits, nullptr, R, d.vocab, d.d, 0, nact, kk, c.s));
    else DLLM_TRY(launch_gemm(c.dtype, p, xn, model->lm_head, logits, R, d.vocab, d.d, nact, kk, c.s));
    DLLM_TRY(t.stop());
  }
  {
    TimedRegion t(c.timing, DLLM_TK_VOCAB, R, c.s);
    DLLM_TRY(t.err);
    DLLM_TRY(launch_conf_kl(logits, state->logits_prev, state->logits_prev_dtype, rp, R, d.vocab, model->mask_id,
                            state->have_prev, state->conf, state->argmax, state->kl, c.ws + c.L.vpart, c.s));
    DLLM_TRY(t.stop());
  }
  if (cfg->lock_kl_eps >= 0.f && state->have_prev)
    DLLM_TRY(launch_lock_update(rp, R, state->conf, state->kl, cfg->lock_kl_eps, cfg->lock_conf_min, state->force,
                                c.s));
  if (cfg->unmask_n > 0) {
    if (cfg->unmask_mode == DLLM_UNMASK_FORCED)
      DLLM_TRY(launch_unmask_forced(state->tokens, state->force, state->argmax, B, S, model->mask_id, cfg->block_lo,
                                    cfg->block_hi, c.s));
    else
      DLLM_TRY(launch_unmask(state->tokens, state->conf, state->argmax, B, S, model->mask_id, cfg->block_lo,
                             cfg->block_hi, cfg->unmask_n, c.s));
  }
  state->bnd_cur = 1 - state->bnd_cur;
  state->have_prev = 1;
  return DLLM_OK;
}

}  // extern "C"
