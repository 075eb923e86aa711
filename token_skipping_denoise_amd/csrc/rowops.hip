// Row-wise kernels: embedding, gather/scatter of active rows, RMSNorm, and the
// reduction epilogues of the split-K GEMMs (RoPE + K/V cache scatter, residual
// add + RMSNorm, SwiGLU).  These are HBM/latency bound: one wavefront per row
// for the row-norm kernels, 16-byte vector accesses throughout.
//
// Sources: partial update of active rows and in-place cache update
// (ES-dLLM summary, technical summary 2.1 item 2); fresh K/V of active rows
// overwrite the cache while other rows keep theirs (SureLock summary 2.1
// items 2-3).  Layer internals (RMSNorm, rotate-half RoPE, SwiGLU) are the
// plain reading of the LLaDA/Dream model family named on the pages.
#include "common.h"
#include "kernels.h"

namespace dllm {

enum RowMode { kEmbed = 0, kGather = 1, kScatter = 2 };

constexpr int kRowThreads = 512;                  // threads of a row-norm workgroup
constexpr int kRowChunks = 1024 / kRowThreads;    // 16-byte chunks per thread: rows up to 1024 chunks

// Sum over the workgroup: butterfly within each wave, then the wave sums in wave order.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) t += red[w];
  return t;
}



// One workgroup per row: copy a row (by token id, gather or scatter) and optionally write
// its RMSNorm * g.  The sum of squares uses the same chunk assignment and reduction order
// as k_resid_norm, so a row normalised here and one normalised there are bit-identical.
template <typename T, int MODE, int NT = kRowThreads>
__global__ __launch_bounds__(NT) void k_rows_norm(const T* __restrict__ src, const int32_t* __restrict__ map,
                                                   int V, int rows, int w, T* __restrict__ dst,
                                                   const T* __restrict__ g, float eps, T* __restrict__ dst_norm,
                                                   T* __restrict__ dst_at_src, uint32_t* chk) {
  using E = Elem<T>;
  constexpr int VE = E::kVec;
  constexpr int CH = 1024 / NT;  // 16-byte chunks per thread
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  long src_row, dst_row;
  if (MODE == kEmbed) {
    int t = map[r];
    if ((t < 0 || t >= V) && threadIdx.x == 0) check_flag(chk, kChkTokenRange);
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);
    src_row = t;
    dst_row = r;
  } else {
    const int pos = map[r];
    if (pos < 0) return;
    src_row = (MODE == kGather) ? pos : r;
    dst_row = (MODE == kGather) ? r : pos;
  }
  const int nchunk = w / VE;
  const uint4* s4 = reinterpret_cast<const uint4*>(src + src_row * (long)w);
  uint4* d4 = dst ? reinterpret_cast<uint4*>(dst + dst_row * (long)w) : nullptr;
  uint4* m4 = dst_at_src ? reinterpret_cast<uint4*>(dst_at_src + src_row * (long)w) : nullptr;  // gather only
  float f[CH][VE];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = threadIdx.x + NT * k;
    if (c >= nchunk) break;
    const uint4 v = s4[c];
    if (d4) d4[c] = v;
    if (m4) m4[c] = v;
    E::unpack(v, f[k]);
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += f[k][e] * f[k][e];
  }
  if (!g) return;
  ss = block_sum<NT>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)w + eps);
  const uint4* g4 = reinterpret_cast<const uint4*>(g);
  uint4* n4 = reinterpret_cast<uint4*>(dst_norm + (long)r * w);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = threadIdx.x + NT * k;
    if (c >= nchunk) break;
    float gf[VE];
    E::unpack(g4[c], gf);
#pragma unroll
    for (int e = 0; e < VE; ++e) f[k][e] = f[k][e] * inv * gf[e];
    n4[c] = E::pack(f[k]);
  }
}

template <int MODE>
static hipError_t rows_norm(int dtype, const void* src, const int32_t* map, int V, int rows, int w, void* dst,
                            const void* g, float eps, void* dst_norm, hipStream_t s, void* dst_at_src = nullptr,
                            uint32_t* chk = nullptr) {
  if (rows <= 0) return hipSuccess;
  if (w / (dtype == 0 ? 4 : 8) > kRowThreads * kRowChunks) return hipErrorInvalidValue;
  dim3 grid(rows), block(kRowThreads);
  if (dtype == 0)
    hipLaunchKernelGGL((k_rows_norm<float, MODE>), grid, block, 0, s, (const float*)src, map, V, rows, w,
                       (float*)dst, (const float*)g, eps, (float*)dst_norm, (float*)dst_at_src, chk);
  else
    hipLaunchKernelGGL((k_rows_norm<bf16, MODE>), grid, block, 0, s, (const bf16*)src, map, V, rows, w,
                       (bf16*)dst, (const bf16*)g, eps, (bf16*)dst_norm, (bf16*)dst_at_src, chk);
  return hipGetLastError();
}

hipError_t launch_embed_norm(int dtype, const void* embed, const int32_t* tokens, int V, int rows, int d,
                             const void* g, float eps, void* x, void* xn, hipStream_t s, uint32_t* chk) {
  return rows_norm<kEmbed>(dtype, embed, tokens, V, rows, d, x, g, eps, xn, s, nullptr, chk);
}
hipError_t launch_gather_norm(int dtype, const void* src, const int32_t* row_pos, int R, int w, void* dst,
                              const void* g, float eps, void* dst_norm, hipStream_t s, void* dst_at_src) {
  return rows_norm<kGather>(dtype, src, row_pos, 0, R, w, dst, g, eps, dst_norm, s, dst_at_src);
}
hipError_t launch_scatter_norm(int dtype, const void* src, const int32_t* row_pos, int R, int w, void* dst,
                               const void* g, float eps, void* dst_norm, hipStream_t s) {
  return rows_norm<kScatter>(dtype, src, row_pos, 0, R, w, dst, g, eps, dst_norm, s);
}

__global__ void k_row_pos(const int32_t* __restrict__ idx, const int32_t* __restrict__ n_active, int B, int S,
                          int k_max, int32_t* __restrict__ row_pos, uint32_t* chk) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B * k_max) return;
  const int b = r / k_max, j = r - b * k_max;
  const int na = n_active[b];
  if (j == 0 && (na < 0 || na > k_max)) check_flag(chk, kChkActiveCount);
  int p = -1;
  if (j < na) {
    const int i = idx[r];
    p = (i >= 0 && i < S) ? b * S + i : -1;
    if (p < 0) check_flag(chk, kChkIndexRange);
    else if (j > 0 && idx[r - 1] >= i) check_flag(chk, kChkIndexOrder);  // live rows ascend strictly
  }
  row_pos[r] = p;
}

hipError_t launch_row_pos(const int32_t* idx, const int32_t* n_active, int B, int S, int k_max, int32_t* row_pos,
                          hipStream_t s, uint32_t* chk) {
  const int n = B * k_max;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_row_pos, dim3((n + 255) / 256), dim3(256), 0, s, idx, n_active, B, S, k_max, row_pos, chk);
  return hipGetLastError();
}

__global__ void k_identity_rows(int B, int S, int32_t* __restrict__ idx, int32_t* __restrict__ n_active,
                                int32_t* __restrict__ row_pos) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < B * S) {
    idx[r] = r % S;
    if (row_pos) row_pos[r] = r;  // b S + i
  }
  if (r < B) n_active[r] = S;
}

hipError_t launch_identity_rows(int B, int S, int32_t* idx, int32_t* n_active, hipStream_t s, int32_t* row_pos) {
  const int n = B * S;
  hipLaunchKernelGGL(k_identity_rows, dim3((n + 255) / 256), dim3(256), 0, s, B, S, idx, n_active, row_pos);
  return hipGetLastError();
}

// ---- GEMM epilogues ----
constexpr int kMaxHalf = 64;  // head dims up to 128

__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int splits, long stride, long off) {
  float v = p[off];
  for (int k = 1; k < splits; ++k) v += p[off + k * stride];
  return v;
}

// Columns of the QKV product: [Q: Hq*D | K: Hkv*D | V: Hkv*D].  A row's work is cut into
// units of four rotation pairs of one Q or K head (columns j..j+3 and j+D/2..j+D/2+3) or four
// V columns; a workgroup of 256 threads takes 256 consecutive units of one row, so a row
// spreads over several workgroups.  Every 16-byte partial load of a thread (all SPLITS of
// them) is issued before any arithmetic: a unit costs one memory round trip.  Rotation
// angles i * theta_j, theta_j = base^(-2j/D), are formed in double and reduced modulo 2 pi
// before the single-precision sine and cosine.
constexpr int kQkvUnitsPerBlock = 256;

template <typename T>
__device__ __forceinline__ void store4(T* p, long off, const float* v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p + off) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    const uint32_t w0 = pack_bf16x2(v[0], v[1]);
    const uint32_t w1 = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p + off) = make_uint2(w0, w1);
  }
}

template <typename T, int SPLITS>
__global__ __launch_bounds__(kQkvUnitsPerBlock) void k_qkv_epilogue(const float* __restrict__ part, long sstride,
                                                                    const int32_t* __restrict__ row_pos, int S, int Hq,
                                                                    int Hkv, int D, double log2_base,
                                                                    T* __restrict__ q, T* __restrict__ kc,
                                                                    T* __restrict__ vc) {
  __shared__ float cs[kMaxHalf], sn[kMaxHalf];
  const int r = blockIdx.x;
  const int pos = row_pos[r];
  if (pos < 0) return;
  const int i = pos % S;
  const int half = D / 2, g4 = half / 4;  // 4-pair groups per head
  const int NQ = Hq * D, NK = Hkv * D, N = NQ + 2 * NK;
  const int ngroups = (Hq + Hkv) * g4;  // rotation units, then V units
  const int u = blockIdx.y * kQkvUnitsPerBlock + threadIdx.x;
  const bool rot = u < ngroups;
  const bool val = !rot && u < ngroups + NK / 4;
  const bool need_angles = blockIdx.y * kQkvUnitsPerBlock < ngroups;  // uniform per block
  if (need_angles) {
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
      const double a = (double)i * exp2(-2.0 * j / (double)D * log2_base);
      const double red = a - 6.283185307179586 * rint(a * 0.15915494309189535);
      float sv, cv;
      sincosf((float)red, &sv, &cv);
      cs[j] = cv;
      sn[j] = sv;
    }
  }
  const float* pr = part + (long)r * N;
  int hh = 0, j0 = 0;
  long c1 = 0, c2 = 0;
  if (rot) {
    hh = u / g4;
    j0 = (u - hh * g4) * 4;
    c1 = hh * D + j0;
    c2 = c1 + half;
  } else if (val) {
    c1 = NQ + NK + (long)(u - ngroups) * 4;
  }
  float4 a[SPLITS], b[SPLITS];
#pragma unroll
  for (int sp = 0; sp < SPLITS; ++sp) {
    if (rot || val) a[sp] = *reinterpret_cast<const float4*>(pr + sp * sstride + c1);
    if (rot) b[sp] = *reinterpret_cast<const float4*>(pr + sp * sstride + c2);
  }
  if (need_angles) __syncthreads();
  if (!rot && !val) return;
  float x1[4] = {0.f, 0.f, 0.f, 0.f}, x2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < SPLITS; ++sp) {
    x1[0] += a[sp].x; x1[1] += a[sp].y; x1[2] += a[sp].z; x1[3] += a[sp].w;
    if (rot) { x2[0] += b[sp].x; x2[1] += b[sp].y; x2[2] += b[sp].z; x2[3] += b[sp].w; }
  }
  if (val) {
    store4(vc, (long)pos * NK + (u - ngroups) * 4, x1);
    return;
  }
  float y1[4], y2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float c = cs[j0 + e], sg = sn[j0 + e];
    y1[e] = x1[e] * c - x2[e] * sg;
    y2[e] = x2[e] * c + x1[e] * sg;
  }
  if (hh < Hq) {
    store4(q, (long)r * NQ + hh * D + j0, y1);
    store4(q, (long)r * NQ + hh * D + j0 + half, y2);
  } else {
    const long o = ((long)pos * Hkv + (hh - Hq)) * D;
    store4(kc, o + j0, y1);
    store4(kc, o + j0 + half, y2);
  }
}

template <typename T>
static hipError_t qkv_epilogue_t(const float* part, int splits, long split_stride, const int32_t* row_pos, int R, int S,
                                 int Hq, int Hkv, int D, double log2_base, void* q, void* kc, void* vc, hipStream_t s) {
  const int units = (Hq + Hkv) * (D / 8) + Hkv * D / 4;
  const dim3 grid(R, (units + kQkvUnitsPerBlock - 1) / kQkvUnitsPerBlock);
  switch (splits) {
#define DLLM_QKV_CASE(SP)                                                                                        \
  case SP:                                                                                                       \
    hipLaunchKernelGGL((k_qkv_epilogue<T, SP>), grid, dim3(kQkvUnitsPerBlock), 0, s, part, split_stride, row_pos, \
                       S, Hq, Hkv, D, log2_base, (T*)q, (T*)kc, (T*)vc);                                         \
    break;
    DLLM_QKV_CASE(1) DLLM_QKV_CASE(2) DLLM_QKV_CASE(4) DLLM_QKV_CASE(8)
#undef DLLM_QKV_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qkv_epilogue(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                               int R, int S, int Hq, int Hkv, int D, float rope_base, void* q, void* kc, void* vc,
                               hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (D / 2 > kMaxHalf || (D / 2) % 4 != 0) return hipErrorInvalidValue;
  const double log2_base = log2((double)rope_base);
  if (dtype == 0) return qkv_epilogue_t<float>(part, splits, split_stride, row_pos, R, S, Hq, Hkv, D, log2_base, q, kc, vc, s);
  return qkv_epilogue_t<bf16>(part, splits, split_stride, row_pos, R, S, Hq, Hkv, D, log2_base, q, kc, vc, s);
}

// One workgroup per row: x += sum(partials) (rounded to storage), then xn = rmsnorm(x) * g.
// Every load of the row is issued up front (values stay in registers), so the row costs
// about one memory round trip.
template <typename T, int SPLITS, int NT = kRowThreads>
__global__ __launch_bounds__(NT) void k_resid_norm(const float* __restrict__ part, int splits_unused, long sstride,
                                                    const int32_t* __restrict__ row_pos, int R, int d,
                                                    T* __restrict__ x, const T* __restrict__ g, float eps,
                                                    T* __restrict__ xn, T* __restrict__ x_scat) {
  using E = Elem<T>;
  constexpr int V = E::kVec;
  constexpr int CH = 1024 / NT;  // 16-byte chunks per thread
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  if (row_pos[r] < 0) return;
  const int nchunk = d / V;
  uint4* x4 = reinterpret_cast<uint4*>(x + (long)r * d);
  uint4* s4 = x_scat ? reinterpret_cast<uint4*>(x_scat + (long)row_pos[r] * d) : nullptr;
  const float* pr = part + (long)r * d;
  float f[CH][V];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = threadIdx.x + NT * k;
    if (c >= nchunk) break;
    E::unpack(x4[c], f[k]);
#pragma unroll
    for (int sp = 0; sp < SPLITS; ++sp) {
      const float4* p4 = reinterpret_cast<const float4*>(pr + sp * sstride + (long)c * V);
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) {
        const float4 a = p4[e4];
        f[k][4 * e4] += a.x;
        f[k][4 * e4 + 1] += a.y;
        f[k][4 * e4 + 2] += a.z;
        f[k][4 * e4 + 3] += a.w;
      }
    }
    const uint4 packed = E::pack(f[k]);
    x4[c] = packed;
    if (s4) s4[c] = packed;
    E::unpack(packed, f[k]);  // the stored (rounded) values feed the norm
#pragma unroll
    for (int e = 0; e < V; ++e) ss += f[k][e] * f[k][e];
  }
  if (!g) return;
  ss = block_sum<NT>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  const uint4* g4 = reinterpret_cast<const uint4*>(g);
  uint4* n4 = reinterpret_cast<uint4*>(xn + (long)r * d);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int c = threadIdx.x + NT * k;
    if (c >= nchunk) break;
    float gf[V];
    E::unpack(g4[c], gf);
#pragma unroll
    for (int e = 0; e < V; ++e) f[k][e] = f[k][e] * inv * gf[e];
    n4[c] = E::pack(f[k]);
  }
}

hipError_t launch_resid_norm(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                             int R, int d, void* x, const void* g, float eps, void* xn, hipStream_t s,
                             void* x_scatter) {
  if (R <= 0) return hipSuccess;
  const int vec = dtype == 0 ? 4 : 8;
  if (d % vec != 0 || d / vec > kRowThreads * kRowChunks) return hipErrorInvalidValue;
#define DLLM_RN(T_, SP_)                                                                              \
  hipLaunchKernelGGL((k_resid_norm<T_, SP_>), dim3(R), dim3(kRowThreads), 0, s, part, splits, split_stride, row_pos, R, d, \
                     (T_*)x, (const T_*)g, eps, (T_*)xn, (T_*)x_scatter)
#define DLLM_RN_SPLITS(T_)                          \
  switch (splits) {                                 \
    case 1: DLLM_RN(T_, 1); break;                  \
    case 2: DLLM_RN(T_, 2); break;                  \
    case 4: DLLM_RN(T_, 4); break;                  \
    case 8: DLLM_RN(T_, 8); break;                  \
    default: return hipErrorInvalidValue;           \
  }
  if (dtype == 0) {
    DLLM_RN_SPLITS(float)
  } else {
    DLLM_RN_SPLITS(bf16)
  }
#undef DLLM_RN_SPLITS
#undef DLLM_RN
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ part, int splits, long sstride,
                                                const int32_t* __restrict__ row_pos, int R, int F, T* __restrict__ h) {
  const long n4 = (long)R * F / 4;
  for (long e4 = blockIdx.x * (long)blockDim.x + threadIdx.x; e4 < n4; e4 += (long)gridDim.x * blockDim.x) {
    const long e = e4 * 4;
    const int r = (int)(e / F);
    if (row_pos[r] < 0) continue;
    const int c = (int)(e - (long)r * F);
    const long base = (long)r * 2 * F + c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float gt = sum_splits(part, splits, sstride, base + t);
      const float up = sum_splits(part, splits, sstride, base + F + t);
      const float sg = gt / (1.0f + expf(-gt));
      Elem<T>::st(h, e + t, sg * up);
    }
  }
}

hipError_t launch_swiglu(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos, int R,
                         int F, void* h, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const long n4 = (long)R * F / 4;
  const int grid = (int)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
  if (dtype == 0)
    hipLaunchKernelGGL(k_swiglu<float>, dim3(grid), dim3(256), 0, s, part, splits, split_stride, row_pos, R, F,
                       (float*)h);
  else
    hipLaunchKernelGGL(k_swiglu<bf16>, dim3(grid), dim3(256), 0, s, part, splits, split_stride, row_pos, R, F,
                       (bf16*)h);
  return hipGetLastError();
}

// dst[r, :] = the split-K partials of row r summed (in split order) and stored in T, for the rows
// with row_pos[r] >= 0: a product's rows in the storage precision of the activations.
template <typename T>
__global__ __launch_bounds__(256) void k_sum_store(const float* __restrict__ part, int splits, long sstride,
                                                   const int32_t* __restrict__ row_pos, int R, int w,
                                                   T* __restrict__ dst) {
  const long n4 = (long)R * w / 4;
  for (long e4 = blockIdx.x * (long)blockDim.x + threadIdx.x; e4 < n4; e4 += (long)gridDim.x * blockDim.x) {
    const long e = e4 * 4;
    const int r = (int)(e / w);
    if (row_pos[r] < 0) continue;
    float4 acc = *reinterpret_cast<const float4*>(part + e);
    for (int k = 1; k < splits; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(part + k * sstride + e);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    Elem<T>::st(dst, e, acc.x);
    Elem<T>::st(dst, e + 1, acc.y);
    Elem<T>::st(dst, e + 2, acc.z);
    Elem<T>::st(dst, e + 3, acc.w);
  }
}

hipError_t launch_sum_store(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                            int R, int w, void* dst, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (w % 4 || split_stride % 4) return hipErrorInvalidValue;
  const long n4 = (long)R * w / 4;
  const int grid = (int)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
  if (dtype == 0)
    hipLaunchKernelGGL(k_sum_store<float>, dim3(grid), dim3(256), 0, s, part, splits, split_stride, row_pos, R, w,
                       (float*)dst);
  else
    hipLaunchKernelGGL(k_sum_store<bf16>, dim3(grid), dim3(256), 0, s, part, splits, split_stride, row_pos, R, w,
                       (bf16*)dst);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

}  // namespace dllm
