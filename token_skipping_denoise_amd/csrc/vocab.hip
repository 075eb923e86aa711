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

__global__ __launch_bounds__(kVT) void k_conf_kl(const float* __restrict__ logits, float* __restrict__ logits_prev,
                                                 const int32_t* __restrict__ row_pos, int V, int exclude_id,
                                                 int have_prev, float* __restrict__ conf, int32_t* __restrict__ argmax,
                                                 float* __restrict__ kl) {
  __shared__ Part sh[kVT];
  const int r = blockIdx.x;
  const int pos = row_pos[r];
  if (pos < 0) return;
  const int tid = threadIdx.x;
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
  const int V4 = ((long)z & 15) == 0 && (zp == nullptr || ((long)zp & 15) == 0) ? V / 4 : 0;
  for (int c = tid; c < V4; c += kVT) {
    const float4 a = reinterpret_cast<const float4*>(z)[c];
    float4 bp = make_float4(0.f, 0.f, 0.f, 0.f);
    if (do_kl) bp = reinterpret_cast<const float4*>(zp)[c];
    if (zp) reinterpret_cast<float4*>(zp)[c] = a;
    take(4 * c + 0, a.x, bp.x);
    take(4 * c + 1, a.y, bp.y);
    take(4 * c + 2, a.z, bp.z);
    take(4 * c + 3, a.w, bp.w);
  }
  for (int v = 4 * V4 + tid; v < V; v += kVT) {
    const float a = z[v];
    const float bp = do_kl ? zp[v] : 0.f;
    if (zp) zp[v] = a;
    take(v, a, bp);
  }
  sh[tid] = p;
  __syncthreads();
  for (int w = kVT / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const Part a = sh[tid], b = sh[tid + w];
      Part c;
      c.m = fmaxf(a.m, b.m);
      c.s = rescale(a.s, a.m, c.m) + rescale(b.s, b.m, c.m);
      c.t = rescale(a.t, a.m, c.m) + rescale(b.t, b.m, c.m);
      c.am = (a.m > b.m) ? a.am : (b.m > a.m ? b.am : min(a.am, b.am));
      c.mp = fmaxf(a.mp, b.mp);
      c.sp = rescale(a.sp, a.mp, c.mp) + rescale(b.sp, b.mp, c.mp);
      sh[tid] = c;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const Part f = sh[0];
    conf[pos] = 1.0f / f.s;
    argmax[pos] = f.am;
    if (kl) {
      if (do_kl) {
        // lse - lse' = (m - m') + log(s / s'): avoids cancelling two O(log V) quantities
        kl[pos] = fmaxf(0.f, f.t / f.s - (f.m - f.mp) - logf(f.s / f.sp));
      } else {
        kl[pos] = INFINITY;
      }
    }
  }
}

hipError_t launch_conf_kl(const float* logits, float* logits_prev, const int32_t* row_pos, int R, int V,
                          int exclude_id, int have_prev, float* conf, int32_t* argmax, float* kl, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_conf_kl, dim3(R), dim3(kVT), 0, s, logits, logits_prev, row_pos, V, exclude_id, have_prev,
                     conf, argmax, kl);
  return hipGetLastError();
}

}  // namespace dllm
