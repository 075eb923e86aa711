// Fused vocabulary pass: confidence, argmax and local KL of each active row.
//
// SureLock (technical summary 2.1 item 1) monitors D = KL(p_t || p_{t-1}) per
// position between successive iterations; ES-dLLM's Eq. 1 reuses the previous
// iteration's confidence.  One workgroup per active row streams its logits
// once (and the row's previous logits once, which it then overwrites), with
// per-thread online max / sum-exp / argmax / KL numerator, combined by a fixed
// tree so the result is deterministic.  HBM bound: 4 V bytes per row without
// KL, 12 V bytes with it.
//
// KL = sum_v p_v (z_v - z'_v) - (lse - lse'), clamped at 0; for identical
// logits the numerator is exactly 0 and both log-sum-exps are computed by the
// same operation sequence, so KL is exactly 0.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int kVT = 256;

struct Part {
  float m, s, t, mp, sp;
  int am;
};

__device__ __forceinline__ float rescale(float s, float m_old, float m_new) {
  return (m_old == -INFINITY) ? 0.f : s * expf(m_old - m_new);
}

__device__ __forceinline__ Part combine(const Part& a, const Part& b) {
  Part c;
  c.m = fmaxf(a.m, b.m);
  c.s = rescale(a.s, a.m, c.m) + rescale(b.s, b.m, c.m);
  c.t = rescale(a.t, a.m, c.m) + rescale(b.t, b.m, c.m);
  c.am = (a.m > b.m) ? a.am : (b.m > a.m ? b.am : min(a.am, b.am));
  c.mp = fmaxf(a.mp, b.mp);
  c.sp = rescale(a.sp, a.mp, c.mp) + rescale(b.sp, b.mp, c.mp);
  return c;
}

__device__ __forceinline__ void finish(const Part& f, int pos, bool do_kl, float* conf, int32_t* argmax, float* kl) {
  conf[pos] = 1.0f / f.s;
  argmax[pos] = f.am;
  if (kl) {
    // lse - lse' = (m - m') + log(s / s'): avoids cancelling two O(log V) quantities
    kl[pos] = do_kl ? fmaxf(0.f, f.t / f.s - (f.m - f.mp) - logf(f.s / f.sp)) : INFINITY;
  }
}

// One workgroup per (row, vocabulary slice).  With nparts == 1 it writes the row's
// statistics; otherwise it writes its slice's partial state to `partial` for k_conf_kl_merge.
__global__ __launch_bounds__(kVT) void k_conf_kl(const float* __restrict__ logits, float* __restrict__ logits_prev,
                                                 const int32_t* __restrict__ row_pos, int V, int exclude_id,
                                                 int have_prev, float* __restrict__ conf, int32_t* __restrict__ argmax,
                                                 float* __restrict__ kl, int nparts, int slice,
                                                 Part* __restrict__ partial) {
  __shared__ Part sh[kVT];
  const int r = blockIdx.x;
  const int pos = row_pos[r];
  if (pos < 0) return;
  const int tid = threadIdx.x;
  const int v0 = blockIdx.y * slice, v1 = min(V, v0 + slice);
  const float* z = logits + (long)r * V;
  float* zp = logits_prev ? logits_prev + (long)pos * V : nullptr;
  const bool do_kl = zp && have_prev;

  Part p{-INFINITY, 0.f, 0.f, -INFINITY, 0.f, 0x7fffffff};
  auto take = [&](int v, float x, float xp) {
    if (v == exclude_id) return;
    if (x > p.m) {
      p.s = rescale(p.s, p.m, x);
      p.t = rescale(p.t, p.m, x);
      p.m = x;
      p.am = v;
    }
    const float e = expf(x - p.m);
    p.s += e;
    if (do_kl) {
      p.t += e * (x - xp);
      if (xp > p.mp) {
        p.sp = rescale(p.sp, p.mp, xp);
        p.mp = xp;
      }
      p.sp += expf(xp - p.mp);
    }
  };
  // 16-byte path when the slice and both rows are 16-byte aligned
  const bool vec = ((((long)(z + v0)) | (zp ? (long)(zp + v0) : 0)) & 15) == 0;
  const int n4 = vec ? (v1 - v0) / 4 : 0;
  for (int c = tid; c < n4; c += kVT) {
    const int v = v0 + 4 * c;
    const float4 a = *reinterpret_cast<const float4*>(z + v);
    float4 bp = make_float4(0.f, 0.f, 0.f, 0.f);
    if (do_kl) bp = *reinterpret_cast<const float4*>(zp + v);
    if (zp) *reinterpret_cast<float4*>(zp + v) = a;
    take(v + 0, a.x, bp.x);
    take(v + 1, a.y, bp.y);
    take(v + 2, a.z, bp.z);
    take(v + 3, a.w, bp.w);
  }
  for (int v = v0 + 4 * n4 + tid; v < v1; v += kVT) {
    const float a = z[v];
    const float bp = do_kl ? zp[v] : 0.f;
    if (zp) zp[v] = a;
    take(v, a, bp);
  }
  sh[tid] = p;
  __syncthreads();
  for (int w = kVT / 2; w > 0; w >>= 1) {
    if (tid < w) sh[tid] = combine(sh[tid], sh[tid + w]);
    __syncthreads();
  }
  if (tid == 0) {
    if (nparts == 1) finish(sh[0], pos, do_kl, conf, argmax, kl);
    else partial[(long)r * nparts + blockIdx.y] = sh[0];
  }
}

// Combine the slices of each row in slice order (deterministic).
__global__ void k_conf_kl_merge(const Part* __restrict__ partial, int nparts, const int32_t* __restrict__ row_pos,
                                int R, int have_prev, int has_prev_buf, float* __restrict__ conf,
                                int32_t* __restrict__ argmax, float* __restrict__ kl) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int pos = row_pos[r];
  if (pos < 0) return;
  Part f = partial[(long)r * nparts];
  for (int k = 1; k < nparts; ++k) f = combine(f, partial[(long)r * nparts + k]);
  finish(f, pos, has_prev_buf && have_prev, conf, argmax, kl);
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

hipError_t launch_conf_kl(const float* logits, float* logits_prev, const int32_t* row_pos, int R, int V,
                          int exclude_id, int have_prev, float* conf, int32_t* argmax, float* kl, void* partial,
                          hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const int parts = partial ? conf_kl_parts(R, V) : 1;  // no scratch: one workgroup per row
  const int slice = ((V + parts - 1) / parts + 3) / 4 * 4;
  hipLaunchKernelGGL(k_conf_kl, dim3(R, parts), dim3(kVT), 0, s, logits, logits_prev, row_pos, V, exclude_id,
                     have_prev, conf, argmax, kl, parts, slice, (Part*)partial);
  if (parts > 1)
    hipLaunchKernelGGL(k_conf_kl_merge, dim3((R + 63) / 64), dim3(64), 0, s, (const Part*)partial, parts, row_pos, R,
                       have_prev, logits_prev != nullptr, conf, argmax, kl);
  return hipGetLastError();
}

}  // namespace dllm
