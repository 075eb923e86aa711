// Bidirectional attention of the active queries over the whole K/V cache.
//
// The model family is non-causal (ES-dLLM summary section 1: every iteration
// processes the full bidirectional context).  Skipped or locked positions are
// not recomputed but stay attendable through the K/V cached when they were
// last computed (ES-dLLM 2.1 item 2; SureLock 2.1 item 3), so the cost is
// O(M_t * N * d) for M_t active rows (SureLock 2.1 item 4).
//
// bf16 kernel (gfx950 MFMA, flash style): a workgroup owns 128 queries of one
// (sequence, KV head) -- the rows x the GQA heads that share that KV head --
// and streams 64-key tiles of K and V through double-buffered LDS (K as
// [key][d], V transposed to [d][key]).  Scores are formed transposed,
// S^T = K Q^T, so each lane holds one query and its online-softmax state;
// the exponentiated scores then serve directly as the B operand of
// O^T += V^T P^T, with the key order inside a fragment chosen to match the
// accumulator layout (any consistent k order gives the same contraction).
//
// fp32 kernel (small fp32 models): one wavefront per (row, head), keys one at
// a time with an online softmax.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------- fp32 ----------------
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ q, const float* __restrict__ kc,
                                                  const float* __restrict__ vc, float* __restrict__ o,
                                                  const int32_t* __restrict__ n_active, int S, int k_max, int Hq,
                                                  int Hkv, int D, float scale) {
  const int r = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int b = r / k_max, j = r - b * k_max;
  if (h >= Hq || j >= n_active[b]) return;
  const int g = Hq / Hkv, hk = h / g;
  const int nd = D / kWave;  // 1 or 2
  float qv[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  for (int t = 0; t < nd; ++t) qv[t] = q[((long)r * Hq + h) * D + lane + t * kWave];
  float m = -INFINITY, l = 0.f;
  for (int key = 0; key < S; ++key) {
    const long base = (((long)b * S + key) * Hkv + hk) * D;
    float part = 0.f;
    for (int t = 0; t < nd; ++t) part += qv[t] * kc[base + lane + t * kWave];
    const float s = wave_sum(part) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn), p = expf(s - mn);
    l = l * corr + p;
    for (int t = 0; t < nd; ++t) acc[t] = acc[t] * corr + p * vc[base + lane + t * kWave];
    m = mn;
  }
  for (int t = 0; t < nd; ++t) o[((long)r * Hq + h) * D + lane + t * kWave] = acc[t] / l;
}

// ---------------- bf16 MFMA ----------------
constexpr int kKT = 64;           // keys per tile
constexpr int kHD = 128;          // head dim
constexpr int kLDK = kHD + 8;     // K tile row stride (elements)
constexpr int kLDV = kKT + 4;     // V^T tile row stride (elements)

// With nsplit > 1 the key tiles are divided among nsplit workgroups (split-KV): each writes
// its unnormalised output and softmax statistics (max, sum, in the exp2 domain) to `part`,
// and k_attn_merge combines them.
__global__ __launch_bounds__(256, 2) void k_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                      const uint16_t* __restrict__ vc, uint16_t* __restrict__ o,
                                                      const int32_t* __restrict__ n_active, int S, int k_max, int Hq,
                                                      int Hkv, float scale_log2e, int nsplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKT * kLDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][kHD * kLDV];
  const int b = blockIdx.z / nsplit, split = blockIdx.z - b * nsplit, hk = blockIdx.y;
  const int g = Hq / Hkv;
  const int nq = n_active[b] * g;
  const int qb0 = blockIdx.x * 128;
  if (qb0 >= nq) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // this lane's query
  const int qi = qb0 + wave * 32 + l32;
  const bool qvalid = qi < nq;
  const int jrow = qvalid ? qi / g : 0, hg = qvalid ? qi - jrow * g : 0;
  const long qrow = (long)b * k_max + jrow;
  const int h = hk * g + hg;
  bf16x8_t qf[kHD / 16];
  {
    const uint16_t* qp = q + (qrow * Hq + h) * kHD + 8 * hi;
#pragma unroll
    for (int t = 0; t < kHD / 16; ++t) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * t) : make_uint4(0, 0, 0, 0);
      qf[t] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // tile loaders: 64 keys x 128 d = 1024 16-byte chunks per tensor, 4 per thread
  uint4 rk[4], rv[4];
  const long kv_row0 = (long)b * S;
  auto load_global = [&](int key0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, key = c >> 4, d0 = (c & 15) * 8;
      const int gk = key0 + key;
      if (gk < S) {
        const long off = ((kv_row0 + gk) * Hkv + hk) * kHD + d0;
        rk[i] = *reinterpret_cast<const uint4*>(kc + off);
        rv[i] = *reinterpret_cast<const uint4*>(vc + off);
      } else {
        rk[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, key = c >> 4, d0 = (c & 15) * 8;
      *reinterpret_cast<uint4*>(&Ks[buf][key * kLDK + d0]) = rk[i];
      const uint32_t w[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[buf][(d0 + 2 * e) * kLDV + key] = (uint16_t)(w[e] & 0xffffu);
        Vt[buf][(d0 + 2 * e + 1) * kLDV + key] = (uint16_t)(w[e] >> 16);
      }
    }
  };

  f32x16_t oacc[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles_all = (S + kKT - 1) / kKT;
  const int t_begin = (int)((long)split * ntiles_all / nsplit), t_end = (int)((long)(split + 1) * ntiles_all / nsplit);
  load_global(t_begin * kKT);
  store_lds(0);
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_global((t + 1) * kKT);

    // S^T for two 32-key blocks
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int ts = 0; ts < kHD / 16; ++ts) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&Ks[buf][(kb * 32 + l32) * kLDK + ts * 16 + 8 * hi]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ts], sacc[kb], 0, 0, 0);
      }
    }
    // scale, mask the tail, online softmax (each query lives in lanes l and l^32)
    const int key0 = t * kKT;
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        float sv = sacc[kb][e] * scale_log2e;
        if (key >= S) sv = -INFINITY;
        sacc[kb][e] = sv;
        mt = fmaxf(mt, sv);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);
    const float corr = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(sacc[kb][e] - m_new);
        sacc[kb][e] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, kWave);
    l_run = l_run * corr + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int kb = s2 >> 1, hf = s2 & 1;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pw[e] = (uint32_t)f2bf(sacc[kb][8 * hf + 2 * e]) | ((uint32_t)f2bf(sacc[kb][8 * hf + 2 * e + 1]) << 16);
      const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      const int kofs = kb * 32 + 16 * hf + 4 * hi;
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db) {
        const uint16_t* vp = &Vt[buf][(db * 32 + l32) * kLDV + kofs];
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hv = *reinterpret_cast<const uint2*>(vp + 8);
        const bf16x8_t afrag = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hv.x, hv.y));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, pfrag, oacc[db], 0, 0, 0);
      }
    }
    if (more) store_lds(buf ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  if (nsplit > 1) {
    // partial layout: [split][row][head][D + 2] = unnormalised O, then (m, l)
    const long n_rows = (long)(gridDim.z / nsplit) * k_max;  // B * k_max
    float* pp = part + (((long)split * n_rows + qrow) * Hq + h) * (kHD + 2);
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * hi;
        *reinterpret_cast<float2*>(pp + d) = make_float2(oacc[db][4 * e4], oacc[db][4 * e4 + 1]);
        *reinterpret_cast<float2*>(pp + d + 2) = make_float2(oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]);
      }
    if (hi == 0) {
      pp[kHD] = m_run;
      pp[kHD + 1] = l_run;
    }
    return;
  }
  const float inv_l = 1.0f / l_run;
  uint16_t* op = o + (qrow * Hq + h) * kHD;
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = db * 32 + 8 * e4 + 4 * hi;
      const uint32_t w0 = (uint32_t)f2bf(oacc[db][4 * e4] * inv_l) | ((uint32_t)f2bf(oacc[db][4 * e4 + 1] * inv_l) << 16);
      const uint32_t w1 = (uint32_t)f2bf(oacc[db][4 * e4 + 2] * inv_l) | ((uint32_t)f2bf(oacc[db][4 * e4 + 3] * inv_l) << 16);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

// Combine split-KV partials: O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, int nsplit, long split_stride,
                                                    const int32_t* __restrict__ n_active, int k_max, int Hq,
                                                    uint16_t* __restrict__ o) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int b = r / k_max, j = r - b * k_max;
  if (j >= n_active[b]) return;
  const float* p0 = part + ((long)r * Hq + h) * (kHD + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, p0[sp * split_stride + kHD]);
  float L = 0.f, acc = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* ps = p0 + sp * split_stride;
    const float w = exp2f(ps[kHD] - M);
    L += ps[kHD + 1] * w;
    acc += ps[d] * w;
  }
  o[((long)r * Hq + h) * kHD + d] = f2bf(acc / L);
}

int attention_splits(int dtype, int B, int S, int k_max, int Hq, int Hkv) {
  if (dtype == 0) return 1;
  const int g = Hq / Hkv;
  const long wgs = (long)((k_max * g + 127) / 128) * Hkv * B;
  const int ntiles = (S + kKT - 1) / kKT;
  int ns = 1;
  while (ns < 4 && wgs * ns < 256 && ntiles / (ns * 2) >= 2) ns *= 2;
  return ns;
}

size_t attention_part_bytes(int dtype, int B, int S, int k_max, int Hq, int Hkv) {
  const int ns = attention_splits(dtype, B, S, k_max, Hq, Hkv);
  return ns > 1 ? (size_t)ns * B * k_max * Hq * (kHD + 2) * sizeof(float) : 0;
}

hipError_t launch_attention(int dtype, const void* q, const void* kc, const void* vc, void* o,
                            const int32_t* n_active, int B, int S, int k_max, int Hq, int Hkv, int D, float* part,
                            hipStream_t s) {
  if (B <= 0 || k_max <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D % kWave != 0 || D > 2 * kWave) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_f32, dim3(B * k_max, (Hq + 3) / 4), dim3(256), 0, s, (const float*)q, (const float*)kc,
                       (const float*)vc, (float*)o, n_active, S, k_max, Hq, Hkv, D, 1.0f / sqrtf((float)D));
    return hipGetLastError();
  }
  if (D != kHD) return hipErrorInvalidValue;
  const int g = Hq / Hkv;
  const int qblocks = (k_max * g + 127) / 128;
  const float scale_log2e = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
  const int ns = attention_splits(dtype, B, S, k_max, Hq, Hkv);
  if (ns > 1 && !part) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_bf16, dim3(qblocks, Hkv, B * ns), dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)kc,
                     (const uint16_t*)vc, (uint16_t*)o, n_active, S, k_max, Hq, Hkv, scale_log2e, ns, part);
  if (ns > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(B * k_max, Hq), dim3(kHD), 0, s, part, ns, (long)B * k_max * Hq * (kHD + 2),
                       n_active, k_max, Hq, (uint16_t*)o);
  return hipGetLastError();
}

}  // namespace dllm
