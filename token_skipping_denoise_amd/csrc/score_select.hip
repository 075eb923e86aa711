// Importance scoring and active-row selection.
//
// Score (ES-dLLM summary, technical summary 2.1 item 1, Eq. 1): a weighted sum
// of the previous iteration's confidence and the relative change of the
// hidden state since the previous iteration; the change may instead be the
// cosine change (dLLM-Cache explainer, section 3), the relative L2 change, or
// the previous local KL (SureLock summary 2.1 item 1).
//
// Selection (ES-dLLM 2.1 item 2: keep the top-k positions; dLLM-Cache
// section 3-4: recompute rows whose similarity is low, at a bounded ratio;
// SureLock 2.1 item 2: locked rows never run again): one workgroup per
// sequence runs an exact radix select over order-preserving 32-bit keys
// (4 passes of 8 bits, LDS histograms), then a stable block-wide compaction
// writes the chosen positions in ascending order.  Ties go to the lower
// index, so the result is unique and bit-reproducible.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace dllm {

enum { kVarL1N = 0, kVarCos = 1, kVarL2Rel = 2, kVarKL = 3, kVarNone = 4 };
enum { kSelTopK = 0, kSelThreshCap = 1, kSelUnlocked = 2 };

// One wavefront per row.  Sums are accumulated per lane in index order and
// combined by a fixed butterfly, so the result is deterministic.
// Change term of one row pair (the whole wave): L1 / sqrt(w) / |b|, |a - b| / |b| or 1 - cos
// (stable form 0.5 || a/|a| - b/|b| ||^2).  With n4 the wave also copies row a there.
// Rows of up to kChunkRegs * 64 chunks (4096 bf16 or 2048 fp32 values) take a path with every
// load of the lane issued before the first use and both rows kept in registers for the cosine
// pass; the per-lane sums run over the same chunks in the same order as the general loop, so
// both paths give bit-identical results.
constexpr int kChunkRegs = 8;

template <typename T>
__device__ __forceinline__ float change_term_regs(const uint4* a4, const uint4* b4, uint4* n4, int w, int var) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int nchunk = w / E::kVec;
  const bool need_rows = (var == kVarL1N || var == kVarCos || var == kVarL2Rel);
  uint4 va[kChunkRegs], vb[kChunkRegs];
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) {
    const int c = lane + kWave * i;
    if (c < nchunk) {
      va[i] = a4[c];
      if (need_rows) vb[i] = b4[c];
    }
  }
  if (n4) {
#pragma unroll
    for (int i = 0; i < kChunkRegs; ++i)
      if (lane + kWave * i < nchunk) n4[lane + kWave * i] = va[i];
  }
  if (!need_rows) return 0.f;
  float l1 = 0.f, l2 = 0.f, na = 0.f, nb = 0.f;
  int diff = 0;
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) {
    if (lane + kWave * i >= nchunk) break;
    float fa[E::kVec], fb[E::kVec];
    E::unpack(va[i], fa);
    E::unpack(vb[i], fb);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) {
      const float dlt = fa[e] - fb[e];
      diff |= (fa[e] != fb[e]);
      l1 += fabsf(dlt);
      l2 += dlt * dlt;
      na += fa[e] * fa[e];
      nb += fb[e] * fb[e];
    }
  }
  l1 = wave_sum(l1);
  l2 = wave_sum(l2);
  na = wave_sum(na);
  nb = wave_sum(nb);
  diff = wave_or(diff);
  if (var == kVarL1N) return (nb == 0.f) ? (diff ? FLT_MAX : 0.f) : l1 / (sqrtf((float)w) * sqrtf(nb));
  if (var == kVarL2Rel) return (nb == 0.f) ? (diff ? FLT_MAX : 0.f) : sqrtf(l2) / sqrtf(nb);
  if (na == 0.f || nb == 0.f) return diff ? FLT_MAX : 0.f;
  const float ia = 1.0f / sqrtf(na), ib = 1.0f / sqrtf(nb);
  float c2 = 0.f;
#pragma unroll
  for (int i = 0; i < kChunkRegs; ++i) {
    if (lane + kWave * i >= nchunk) break;
    float fa[E::kVec], fb[E::kVec];
    E::unpack(va[i], fa);
    E::unpack(vb[i], fb);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) {
      const float t = fa[e] * ia - fb[e] * ib;
      c2 += t * t;
    }
  }
  return 0.5f * wave_sum(c2);
}

template <typename T>
__device__ __forceinline__ float change_term(const uint4* a4, const uint4* b4, uint4* n4, int w, int var) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int nchunk = w / E::kVec;
  if (nchunk <= kChunkRegs * kWave) return change_term_regs<T>(a4, b4, n4, w, var);
  float l1 = 0.f, l2 = 0.f, na = 0.f, nb = 0.f;
  int diff = 0;
  const bool need_rows = (var == kVarL1N || var == kVarCos || var == kVarL2Rel);
  if (need_rows || n4) {
    for (int c = lane; c < nchunk; c += kWave) {
      const uint4 va = a4[c];
      if (n4) n4[c] = va;
      if (!need_rows) continue;
      const uint4 vb = b4[c];
      float fa[E::kVec], fb[E::kVec];
      E::unpack(va, fa);
      E::unpack(vb, fb);
#pragma unroll
      for (int e = 0; e < E::kVec; ++e) {
        const float dlt = fa[e] - fb[e];
        diff |= (fa[e] != fb[e]);
        l1 += fabsf(dlt);
        l2 += dlt * dlt;
        na += fa[e] * fa[e];
        nb += fb[e] * fb[e];
      }
    }
  }
  if (!need_rows) return 0.f;
  l1 = wave_sum(l1);
  l2 = wave_sum(l2);
  na = wave_sum(na);
  nb = wave_sum(nb);
  diff = wave_or(diff);
  if (var == kVarL1N) return (nb == 0.f) ? (diff ? FLT_MAX : 0.f) : l1 / (sqrtf((float)w) * sqrtf(nb));
  if (var == kVarL2Rel) return (nb == 0.f) ? (diff ? FLT_MAX : 0.f) : sqrtf(l2) / sqrtf(nb);
  if (na == 0.f || nb == 0.f) return diff ? FLT_MAX : 0.f;
  const float ia = 1.0f / sqrtf(na), ib = 1.0f / sqrtf(nb);
  float c2 = 0.f;
  for (int c = lane; c < nchunk; c += kWave) {
    float fa[E::kVec], fb[E::kVec];
    E::unpack(a4[c], fa);
    E::unpack(b4[c], fb);
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) {
      const float t = fa[e] * ia - fb[e] * ib;
      c2 += t * t;
    }
  }
  return 0.5f * wave_sum(c2);
}

__device__ __forceinline__ float importance(float c, float psi, float alpha, int conf_inverted) {
  const float phi = conf_inverted ? 1.0f - c : c;
  return alpha * phi + (1.0f - alpha) * psi;
}

// ES-dLLM Eq. 1 (and variants) for every position: one wave per row.
template <typename T>
__global__ __launch_bounds__(64) void k_score(const T* __restrict__ h_cur, const T* __restrict__ h_prev,
                                              T* __restrict__ h_next, const float* __restrict__ conf_prev,
                                              const float* __restrict__ kl_prev, int rows, int w, float alpha,
                                              int conf_inverted, int var, float* __restrict__ score) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x;  // one row per single-wave workgroup: the rows spread over every CU
  if (r >= rows) return;
  const uint4* a4 = reinterpret_cast<const uint4*>(h_cur + (long)r * w);
  const uint4* b4 = reinterpret_cast<const uint4*>(h_prev + (long)r * w);
  uint4* n4 = h_next ? reinterpret_cast<uint4*>(h_next + (long)r * w) : nullptr;
  float psi = change_term<T>(a4, b4, n4, w, var == kVarKL ? kVarNone : var);
  if (var == kVarKL) psi = kl_prev[r];
  if (lane == 0) score[r] = importance(conf_prev[r], psi, alpha, conf_inverted);
}

// Nested boundary: the same score for the active rows only, from the row's current hidden state
// (x_act row r) and the per-layer cache at its position p = row_pos[r].  Marks the active
// positions as candidates in force_nested (the caller set every position to excluded first;
// a forced row stays forced) and records the row of each active position in row_of.
template <typename T>
__global__ __launch_bounds__(256) void k_score_rows(const T* __restrict__ x_act, const int32_t* __restrict__ row_pos,
                                                    const T* __restrict__ h_cache, const float* __restrict__ conf_prev,
                                                    const float* __restrict__ kl_prev,
                                                    const uint8_t* __restrict__ force, int R, int w, float alpha,
                                                    int conf_inverted, int var, float* __restrict__ score,
                                                    uint8_t* __restrict__ force_nested, int32_t* __restrict__ row_of) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int p = row_pos[r];
  if (p < 0) return;
  const uint4* a4 = reinterpret_cast<const uint4*>(x_act + (long)r * w);
  const uint4* b4 = reinterpret_cast<const uint4*>(h_cache + (long)p * w);
  float psi = change_term<T>(a4, b4, nullptr, w, var == kVarKL ? kVarNone : var);
  if (var == kVarKL) psi = kl_prev[p];
  if (lane == 0) {
    score[p] = importance(conf_prev[p], psi, alpha, conf_inverted);
    force_nested[p] = (force && force[p] == 1) ? 1 : 0;
    row_of[p] = r;
  }
}

__global__ void k_fill_excluded(uint8_t* __restrict__ force_nested, int32_t* __restrict__ row_of, long n) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (i >= n) return;
  force_nested[i] = 2;
  row_of[i] = -1;
}

// old_row[r] = row_of[row_pos[r]] for the rows of the narrowed set (-1 for dead rows)
__global__ void k_compose_rows(const int32_t* __restrict__ row_pos, const int32_t* __restrict__ row_of, int R,
                               int32_t* __restrict__ old_row) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int p = row_pos[r];
  old_row[r] = p < 0 ? -1 : row_of[p];
}

hipError_t launch_score(int dtype, const void* h_cur, const void* h_prev, void* h_next, const float* conf_prev,
                        const float* kl_prev, const uint8_t* force, int rows, int width, float alpha,
                        int conf_inverted, int var, float* score, hipStream_t s) {
  (void)force;  // forced and excluded rows are handled by the selection
  if (rows <= 0) return hipSuccess;
  dim3 grid(rows), block(64);
  if (dtype == 0)
    hipLaunchKernelGGL(k_score<float>, grid, block, 0, s, (const float*)h_cur, (const float*)h_prev, (float*)h_next,
                       conf_prev, kl_prev, rows, width, alpha, conf_inverted, var, score);
  else
    hipLaunchKernelGGL(k_score<bf16>, grid, block, 0, s, (const bf16*)h_cur, (const bf16*)h_prev, (bf16*)h_next,
                       conf_prev, kl_prev, rows, width, alpha, conf_inverted, var, score);
  return hipGetLastError();
}

hipError_t launch_score_rows(int dtype, const void* x_act, const int32_t* row_pos, int R, const void* h_cache,
                             const float* conf_prev, const float* kl_prev, const uint8_t* force, long positions,
                             int width, float alpha, int conf_inverted, int var, float* score, uint8_t* force_nested,
                             int32_t* row_of, hipStream_t s) {
  if (positions > 0)
    hipLaunchKernelGGL(k_fill_excluded, dim3((unsigned)((positions + 255) / 256)), dim3(256), 0, s, force_nested,
                       row_of, positions);
  if (R <= 0) return hipGetLastError();
  dim3 grid((R + 3) / 4), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(k_score_rows<float>, grid, block, 0, s, (const float*)x_act, row_pos, (const float*)h_cache,
                       conf_prev, kl_prev, force, R, width, alpha, conf_inverted, var, score, force_nested, row_of);
  else
    hipLaunchKernelGGL(k_score_rows<bf16>, grid, block, 0, s, (const bf16*)x_act, row_pos, (const bf16*)h_cache,
                       conf_prev, kl_prev, force, R, width, alpha, conf_inverted, var, score, force_nested, row_of);
  return hipGetLastError();
}

hipError_t launch_compose_rows(const int32_t* row_pos, const int32_t* row_of, int R, int32_t* old_row, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_compose_rows, dim3((R + 255) / 256), dim3(256), 0, s, row_pos, row_of, R, old_row);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelCache = 4096;  // positions whose keys a selection keeps in LDS
constexpr int kSelWaves = kSelThreads / kWave;

// Order-preserving key: larger key = selected earlier.  NaN -> 0 (below -inf),
// -0 -> +0, forced rows -> 0xFFFFFFFF (above +inf).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct BlockScan {
  int wave_tot[kSelWaves];
};

// Exclusive prefix count of `flag` over the block (thread order) and the block total.
__device__ __forceinline__ int block_excl_count(bool flag, BlockScan& sh, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) sh.wave_tot[wv] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    const int t = sh.wave_tot[i];
    if (i < wv) before += t;
    total += t;
  }
  __syncthreads();
  return before + in_wave;
}

__device__ __forceinline__ int block_count(bool flag, BlockScan& sh) {
  int total;
  (void)block_excl_count(flag, sh, total);
  return total;
}

__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ score,
                                                        const uint8_t* __restrict__ force, int S, int sel, int k,
                                                        float tau, int k_max, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ n_active, int32_t* __restrict__ row_pos) {
  __shared__ BlockScan sh;
  __shared__ int hist[256];
  __shared__ int bcast[2];
  // keys of up to kSelCache positions, read from memory once (the radix passes and the
  // compaction then read LDS); a non-candidate position is marked in cflag
  __shared__ uint32_t kkey[kSelCache];
  __shared__ uint8_t kcand[kSelCache];
  const int b = blockIdx.x;
  const float* sc = score + (long)b * S;
  const uint8_t* fo = force ? force + (long)b * S : nullptr;
  const int tid = threadIdx.x;
  const bool cached = S <= kSelCache;
  // candidate flag and key of position i: f = 2 excluded, f = 1 forced (largest key)
  auto cand_key = [&](int i, uint32_t& key) -> bool {
    if (cached) {
      key = kkey[i];
      return kcand[i] != 0;
    }
    const int f = fo ? fo[i] : 0;
    key = (f == 1) ? 0xffffffffu : score_key(sc[i]);
    return f != 2;
  };

  // candidates and threshold qualifiers
  int n_cand = 0, n_q = 0;
  for (int i0 = 0; i0 < S; i0 += kSelThreads) {
    const int i = i0 + tid;
    bool cand = false, q = false;
    if (i < S) {
      const int f = fo ? fo[i] : 0;
      const float v = sc[i];
      cand = (f != 2);
      q = cand && (f == 1 || v > tau);
      if (cached) {
        kkey[i] = (f == 1) ? 0xffffffffu : score_key(v);
        kcand[i] = cand ? 1 : 0;
      }
    }
    n_cand += block_count(cand, sh);  // its barrier also publishes the cached keys
    n_q += block_count(q, sh);
  }
  int k_eff = (sel == kSelUnlocked) ? n_cand : (sel == kSelThreshCap ? min(k, n_q) : min(k, n_cand));
  if (k_eff < 0) k_eff = 0;

  // radix select of the k_eff-th largest key
  uint32_t kth = 0u;
  int take_eq = 0;  // how many keys equal to kth are taken (lowest indices first)
  const bool take_all = (k_eff >= n_cand);
  if (!take_all && k_eff > 0) {
    uint32_t prefix = 0u, hmask = 0u;
    int remaining = k_eff;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int t = tid; t < 256; t += kSelThreads) hist[t] = 0;
      __syncthreads();
      for (int i = tid; i < S; i += kSelThreads) {
        uint32_t key;
        if (!cand_key(i, key)) continue;
        if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l owns bins 4l..4l+3; find the bin where the count from the top reaches `remaining`
        int own = hist[4 * tid] + hist[4 * tid + 1] + hist[4 * tid + 2] + hist[4 * tid + 3];
        int above = own;  // inclusive suffix sum over lanes >= tid
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int v = __shfl_down(above, o, kWave);
          if (tid + o < kWave) above += v;
        }
        int acc = above - own;  // keys in bins above this lane's bins
        for (int dgt = 4 * tid + 3; dgt >= 4 * tid; --dgt) {
          const int hcount = hist[dgt];
          if (acc < remaining && acc + hcount >= remaining) {
            bcast[0] = dgt;
            bcast[1] = acc;
          }
          acc += hcount;
        }
      }
      __syncthreads();
      const int dgt = bcast[0];
      remaining -= bcast[1];
      prefix |= (uint32_t)dgt << shift;
      hmask |= 0xffu << shift;
      __syncthreads();
    }
    kth = prefix;
    take_eq = remaining;
  }

  // stable compaction in ascending index order
  int carry_eq = 0, carry_sel = 0;
  int32_t* out = idx + (long)b * k_max;
  int32_t* rpo = row_pos ? row_pos + (long)b * k_max : nullptr;  // b S + i beside each index
  for (int i0 = 0; i0 < S; i0 += kSelThreads) {
    const int i = i0 + tid;
    bool gt = false, eq = false;
    if (i < S) {
      uint32_t key;
      if (cand_key(i, key)) {
        if (take_all) {
          gt = true;
        } else if (k_eff > 0) {
          gt = key > kth;
          eq = key == kth;
        }
      }
    }
    int tot_eq;
    const int eq_rank = carry_eq + block_excl_count(eq, sh, tot_eq);
    const bool flag = gt || (eq && eq_rank < take_eq);
    int tot_sel;
    const int opos = carry_sel + block_excl_count(flag, sh, tot_sel);
    if (flag && opos < k_max) {
      out[opos] = i;
      if (rpo) rpo[opos] = b * S + i;
    }
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  const int n = min(carry_sel, k_max);
  for (int j = n + tid; j < k_max; j += kSelThreads) {
    out[j] = -1;
    if (rpo) rpo[j] = -1;
  }
  if (tid == 0) n_active[b] = n;
}

hipError_t launch_select(const float* score, const uint8_t* force, int B, int S, int sel, int k, float tau,
                         int k_max, int32_t* idx, int32_t* n_active, hipStream_t s, int32_t* row_pos) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_select, dim3(B), dim3(kSelThreads), 0, s, score, force, S, sel, k, tau, k_max, idx, n_active,
                     row_pos);
  return hipGetLastError();
}

}  // namespace dllm
