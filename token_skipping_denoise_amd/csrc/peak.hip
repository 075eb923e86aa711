// Achievable-peak probes, the measured denominators beside the datasheet ones: a device copy
// and a read-only stream (HBM), and a loop of independent v_mfma_f32_32x32x16_bf16 on register
// operands (the matrix cores with no memory traffic).  Used by the benchmark only; nothing on the denoising
// path calls them.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kProbeUnroll = 4;       // independent 16-byte loads in flight per thread
constexpr int kStreamBlocks = 512;    // 2 workgroups of 256 threads per CU (best of a sweep)

// Grid-stride copy of nchunk chunks of 256 x 4 16-byte elements (each read once, written once).
__global__ __launch_bounds__(256) void k_copy_probe(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                    long nchunk) {
  for (long c = blockIdx.x; c < nchunk; c += gridDim.x) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[(c * kProbeUnroll + u) * 256 + threadIdx.x];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) dst[(c * kProbeUnroll + u) * 256 + threadIdx.x] = v[u];
  }
}

// Grid-stride nontemporal read of the same chunks; the words are folded by xor and stored only
// in a case the fold cannot be known to avoid, so the loads are kept.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4_t* __restrict__ src, long nchunk,
                                                    unsigned* __restrict__ sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (long c = blockIdx.x; c < nchunk; c += gridDim.x) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + (c * kProbeUnroll + u) * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  const unsigned f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (f == 0x9e3779b9u) sink[blockIdx.x * 256 + threadIdx.x] = f;
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
  constexpr long kChunk = 256L * kProbeUnroll * 16;  // bytes per chunk
  if (kind == 0) {
    const long nchunk = (long)(bytes / 2 / kChunk);
    const long half = nchunk * kChunk / 16;
    for (int i = 0; i < iters; ++i)
      hipLaunchKernelGGL(k_copy_probe, dim3(kStreamBlocks), dim3(256), 0, s, (const uint4*)buf, (uint4*)buf + half,
                         nchunk);
    *work = 2.0 * (double)nchunk * kChunk * iters;  // bytes read + written
  } else if (kind == 2) {
    // the sink (one word per thread) takes the first bytes; the stream reads the rest
    const size_t sink_bytes = (size_t)kStreamBlocks * 256 * sizeof(unsigned);
    const long nchunk = (long)((bytes - sink_bytes) / kChunk);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>((const char*)buf + sink_bytes);
    for (int i = 0; i < iters; ++i)
      hipLaunchKernelGGL(k_read_probe, dim3(kStreamBlocks), dim3(256), 0, s, src, nchunk, (unsigned*)buf);
    *work = (double)nchunk * kChunk * iters;  // bytes read
  } else {
    hipLaunchKernelGGL(k_mfma_probe, dim3(kProbeBlocks), dim3(256), 0, s, (float*)buf, iters);
    *work = (double)kProbeBlocks * 4 /* waves */ * 4 /* chains */ * (double)iters * 2.0 * 32 * 32 * 16;
  }
  return hipGetLastError();
}

}  // namespace dllm
