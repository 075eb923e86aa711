// Fused vocabulary pass: confidence, argmax and local KL of each active row.
//
// SureLock (technical summary 2.1 item 1) monitors D = KL(p_t || p_{t-1}) per
// position between successive iterations; ES-dLLM's Eq. 1 reuses the previous
// iteration's confidence.  One workgroup per active row streams its logits
// once (and the row's previous logits once, which it then overwrites), with
// per-thread online max / sum-exp / argmax / KL numerator, combined by a fixed
// tree so the result is deterministic.  HBM bound: 4 V bytes per row without
// KL, 12 V bytes with an fp32 state, 8 V with a bf16 state.
//
// KL = sum_v p_v (z_v - z'_v) - (lse - lse'), clamped at 0; for identical
// logits the numerator is exactly 0 and both log-sum-exps are computed by the
// same operation sequence, so KL is exactly 0.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kVT = 256;

// Online state of a vocabulary slice: max / sum-exp / argmax of the logits (m, s, am); of the
// logits the KL compares (mk, sk, with the KL numerator t relative to mk); of the previous
// logits (mp, sp).  With an fp32 KL state the compared logits are the logits themselves, so
// (mk, sk) are not kept and t is relative to m.
struct Part {
  float m, s, mk, sk, t, mp, sp;
  int am;
};

// e^x as 2^(x log2 e) on the hardware exp2: one multiply-add and one transcendental per
// element, so the pass stays bound by memory rather than by the exponentials
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float rescale(float s, float m_old, float m_new) {
  return (m_old == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m_old - m_new) * kLog2e);
}

// e^(x - m) with m2 = m log2 e computed once per change of m
__device__ __forceinline__ float exp_from(float x, float m2) { return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -m2)); }

// round to bf16 (RNE, the hardware conversion) and back
__device__ __forceinline__ float round_bf16(float x) { return __uint_as_float(pack_bf16x2(x, 0.f) << 16); }

template <bool BF>
__device__ __forceinline__ Part combine(const Part& a, const Part& b) {
  Part c;
  c.m = fmaxf(a.m, b.m);
  c.s = rescale(a.s, a.m, c.m) + rescale(b.s, b.m, c.m);
  c.am = (a.m > b.m) ? a.am : (b.m > a.m ? b.am : min(a.am, b.am));
  if (BF) {
    c.mk = fmaxf(a.mk, b.mk);
    c.sk = rescale(a.sk, a.mk, c.mk) + rescale(b.sk, b.mk, c.mk);
    c.t = rescale(a.t, a.mk, c.mk) + rescale(b.t, b.mk, c.mk);
  } else {
    c.mk = c.sk = 0.f;
    c.t = rescale(a.t, a.m, c.m) + rescale(b.t, b.m, c.m);
  }
  c.mp = fmaxf(a.mp, b.mp);
  c.sp = rescale(a.sp, a.mp, c.mp) + rescale(b.sp, b.mp, c.mp);
  return c;
}

template <bool BF>
__device__ __forceinline__ void finish(const Part& f, int pos, bool do_kl, float* conf, int32_t* argmax, float* kl) {
  conf[pos] = 1.0f / f.s;
  argmax[pos] = f.am;
  if (kl) {
    // lse - lse' = (m - m') + log(s / s'): avoids cancelling two O(log V) quantities
    const float mk = BF ? f.mk : f.m, sk = BF ? f.sk : f.s;
    kl[pos] = do_kl ? fmaxf(0.f, f.t / sk - (mk - f.mp) - logf(sk / f.sp)) : INFINITY;
  }
}

// Previous-logit state: fp32, or bf16 (RNE) with the KL taken between the bf16-rounded current
// logits and the stored ones (identical logits still give exactly 0).
template <typename P>
struct PrevIO;
template <>
struct PrevIO<float> {
  static constexpr bool kBF = false;
  __device__ static __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static __forceinline__ void st4(float* p, float4 a) { *reinterpret_cast<float4*>(p) = a; }
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float a) { *p = a; }
};
template <>
struct PrevIO<uint16_t> {
  static constexpr bool kBF = true;
  __device__ static __forceinline__ float4 ld4(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf2f((uint16_t)(w.x & 0xffff)), bf2f((uint16_t)(w.x >> 16)), bf2f((uint16_t)(w.y & 0xffff)),
                       bf2f((uint16_t)(w.y >> 16)));
  }
  __device__ static __forceinline__ void st4(uint16_t* p, float4 a) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
  }
  __device__ static __forceinline__ float ld(const uint16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void st(uint16_t* p, float a) { *p = (uint16_t)(pack_bf16x2(a, 0.f) & 0xffff); }
};

// One workgroup per (row, vocabulary slice).  With nparts == 1 it writes the row's
// statistics; otherwise it writes its slice's partial state to `partial` for k_conf_kl_merge.
template <typename P>
__global__ __launch_bounds__(kVT) void k_conf_kl(const float* __restrict__ logits, P* __restrict__ logits_prev,
                                                 const int32_t* __restrict__ row_pos, int V, int exclude_id,
                                                 int have_prev, float* __restrict__ conf, int32_t* __restrict__ argmax,
                                                 float* __restrict__ kl, int nparts, int slice,
                                                 Part* __restrict__ partial) {
  using IO = PrevIO<P>;
  constexpr bool BF = IO::kBF;
  __shared__ Part sh[kVT];
  const int r = blockIdx.x;
  const int pos = row_pos[r];
  if (pos < 0) return;
  const int tid = threadIdx.x;
  const int v0 = blockIdx.y * slice, v1 = min(V, v0 + slice);
  const float* z = logits + (long)r * V;
  P* zp = logits_prev ? logits_prev + (long)pos * V : nullptr;
  const bool do_kl = zp && have_prev;

  Part p{-INFINITY, 0.f, -INFINITY, 0.f, 0.f, -INFINITY, 0.f, 0x7fffffff};
  float m2 = -INFINITY, mk2 = -INFINITY, mp2 = -INFINITY;  // the running maxima times log2 e
  auto take = [&](int v, float x, float xp) {
    if (v == exclude_id) return;
    if (x > p.m) {
      p.s = rescale(p.s, p.m, x);
      if (!BF) p.t = rescale(p.t, p.m, x);
      p.m = x;
      m2 = x * kLog2e;
      p.am = v;
    }
    const float e = exp_from(x, m2);
    p.s += e;
    if (do_kl) {
      if (BF) {
        const float xk = round_bf16(x);
        if (xk > p.mk) {
          p.sk = rescale(p.sk, p.mk, xk);
          p.t = rescale(p.t, p.mk, xk);
          p.mk = xk;
          mk2 = xk * kLog2e;
        }
        const float ek = exp_from(xk, mk2);
        p.sk += ek;
        p.t += ek * (xk - xp);
      } else {
        p.t += e * (x - xp);
      }
      if (xp > p.mp) {
        p.sp = rescale(p.sp, p.mp, xp);
        p.mp = xp;
        mp2 = xp * kLog2e;
      }
      p.sp += exp_from(xp, mp2);
    }
  };
  // vector path (4 logits per access) when the slice and both rows are aligned for it
  const bool vec = ((((long)(z + v0)) & 15) | (zp ? ((long)(zp + v0) & (4 * sizeof(P) - 1)) : 0)) == 0;
  const int n4 = vec ? (v1 - v0) / 4 : 0;
  for (int c = tid; c < n4; c += kVT) {
    const int v = v0 + 4 * c;
    const float4 a = *reinterpret_cast<const float4*>(z + v);
    float4 bp = make_float4(0.f, 0.f, 0.f, 0.f);
    if (do_kl) bp = IO::ld4(zp + v);
    if (zp) IO::st4(zp + v, a);
    take(v + 0, a.x, bp.x);
    take(v + 1, a.y, bp.y);
    take(v + 2, a.z, bp.z);
    take(v + 3, a.w, bp.w);
  }
  for (int v = v0 + 4 * n4 + tid; v < v1; v += kVT) {
    const float a = z[v];
    const float bp = do_kl ? IO::ld(zp + v) : 0.f;
    if (zp) IO::st(zp + v, a);
    take(v, a, bp);
  }
  sh[tid] = p;
  __syncthreads();
  for (int w = kVT / 2; w > 0; w >>= 1) {
    if (tid < w) sh[tid] = combine<BF>(sh[tid], sh[tid + w]);
    __syncthreads();
  }
  if (tid == 0) {
    if (nparts == 1) finish<BF>(sh[0], pos, do_kl, conf, argmax, kl);
    else partial[(long)r * nparts + blockIdx.y] = sh[0];
  }
}

// Combine the slices of each row in slice order (deterministic).
template <bool BF>
__global__ void k_conf_kl_merge(const Part* __restrict__ partial, int nparts, const int32_t* __restrict__ row_pos,
                                int R, int have_prev, int has_prev_buf, float* __restrict__ conf,
                                int32_t* __restrict__ argmax, float* __restrict__ kl) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int pos = row_pos[r];
  if (pos < 0) return;
  Part f = partial[(long)r * nparts];
  for (int k = 1; k < nparts; ++k) f = combine<BF>(f, partial[(long)r * nparts + k]);
  finish<BF>(f, pos, has_prev_buf && have_prev, conf, argmax, kl);
}

int conf_kl_parts(int R, int V) {
  int parts = 1;
  while (parts < 32 && (long)R * parts < 2048 && V / (parts * 2) >= 4096) parts *= 2;
  return parts;
}

size_t conf_kl_part_bytes(int R, int V) {
  const int parts = conf_kl_parts(R, V);
  return parts > 1 ? (size_t)R * parts * sizeof(Part) : 0;
}

template <typename P>
static hipError_t conf_kl_t(const float* logits, P* logits_prev, const int32_t* row_pos, int R, int V, int exclude_id,
                            int have_prev, float* conf, int32_t* argmax, float* kl, void* partial, hipStream_t s) {
  const int parts = partial ? conf_kl_parts(R, V) : 1;  // no scratch: one workgroup per row
  const int slice = ((V + parts - 1) / parts + 3) / 4 * 4;
  hipLaunchKernelGGL(k_conf_kl<P>, dim3(R, parts), dim3(kVT), 0, s, logits, logits_prev, row_pos, V, exclude_id,
                     have_prev, conf, argmax, kl, parts, slice, (Part*)partial);
  if (parts > 1)
    hipLaunchKernelGGL(k_conf_kl_merge<PrevIO<P>::kBF>, dim3((R + 63) / 64), dim3(64), 0, s, (const Part*)partial,
                       parts, row_pos, R, have_prev, logits_prev != nullptr, conf, argmax, kl);
  return hipGetLastError();
}

hipError_t launch_conf_kl(const float* logits, void* logits_prev, int prev_dtype, const int32_t* row_pos, int R,
                          int V, int exclude_id, int have_prev, float* conf, int32_t* argmax, float* kl, void* partial,
                          hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (prev_dtype == 1)  // bf16 state
    return conf_kl_t(logits, (uint16_t*)logits_prev, row_pos, R, V, exclude_id, have_prev, conf, argmax, kl, partial, s);
  return conf_kl_t(logits, (float*)logits_prev, row_pos, R, V, exclude_id, have_prev, conf, argmax, kl, partial, s);
}

}  // namespace dllm
