// Achievable-peak probes, the measured denominators beside the datasheet ones: a device copy
// (HBM streaming) and a loop of independent v_mfma_f32_32x32x16_bf16 on register operands (the
// matrix cores with no memory traffic).  Used by the benchmark only; nothing on the denoising
// path calls them.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Grid-stride copy of n 16-byte chunks (each element read once and written once).
__global__ __launch_bounds__(256) void k_copy_probe(const uint4* __restrict__ src, uint4* __restrict__ dst, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) dst[i] = src[i];
}

// Every wave runs 4 independent accumulator chains of `iters` MFMAs each.  The operands come from
// the thread index, so the compiler cannot fold them; a lane stores only when its sums hit a
// value they cannot reach, so the work is kept without memory traffic.
__global__ __launch_bounds__(256) void k_mfma_probe(float* __restrict__ sink, int iters) {
  const int t = threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((t + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)((t * 3 + e) & 7));
  }
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == -1.0f) sink[blockIdx.x * blockDim.x + t] = s;
}

constexpr int kProbeBlocks = 2048;  // 8 workgroups of 4 waves per CU

hipError_t launch_peak_probe(int kind, void* buf, size_t bytes, int iters, double* work, hipStream_t s) {
  if (kind == 0) {
    const long n = (long)(bytes / 2 / 16);
    for (int i = 0; i < iters; ++i)
      hipLaunchKernelGGL(k_copy_probe, dim3(4096), dim3(256), 0, s, (const uint4*)buf, (uint4*)buf + n, n);
    *work = 2.0 * 16.0 * (double)n * iters;  // bytes read + written
  } else {
    hipLaunchKernelGGL(k_mfma_probe, dim3(kProbeBlocks), dim3(256), 0, s, (float*)buf, iters);
    *work = (double)kProbeBlocks * 4 /* waves */ * 4 /* chains */ * (double)iters * 2.0 * 32 * 32 * 16;
  }
  return hipGetLastError();
}

}  // namespace dllm
