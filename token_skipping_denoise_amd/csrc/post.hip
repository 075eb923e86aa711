// Post-step updates that stay on the device (no host synchronisation).
//
// * SureLock lock rule (technical summary 2.1 item 1): a recomputed position
//   locks once its local KL is at or below epsilon and its confidence exceeds
//   the optional minimum; locking is permanent.
// * Confidence unmasking (ES-dLLM summary section 1; SureLock section 1): the
//   n most confident masked positions of the current block receive their
//   argmax token; ties go to the lower position.
// * Planned unmasking (DUS summary, technical summary section 2): the masked
//   positions that a dilated schedule assigns to this round (marked FORCE_ON)
//   receive their argmax token.
#include "common.h"
#include "kernels.h"

namespace dllm {

__global__ void k_lock_update(const int32_t* __restrict__ row_pos, int R, const float* __restrict__ conf,
                              const float* __restrict__ kl, float eps, float conf_min, uint8_t* __restrict__ force) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int pos = row_pos[r];
  if (pos < 0) return;
  if (kl[pos] <= eps && conf[pos] > conf_min) force[pos] = 2;
}

hipError_t launch_lock_update(const int32_t* row_pos, int R, const float* conf, const float* kl, float eps,
                              float conf_min, uint8_t* force, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lock_update, dim3((R + 255) / 256), dim3(256), 0, s, row_pos, R, conf, kl, eps, conf_min, force);
  return hipGetLastError();
}

constexpr int kUT = 256;
constexpr int kMaxUnmask = 256;

// One workgroup per sequence; n rounds of a block-wide arg-max over (conf desc, position asc).
__global__ __launch_bounds__(kUT) void k_unmask(int32_t* __restrict__ tokens, const float* __restrict__ conf,
                                                const int32_t* __restrict__ argmax, int S, int mask_id, int lo, int hi,
                                                int n) {
  __shared__ int chosen[kMaxUnmask];
  __shared__ float bc[kUT];
  __shared__ int bi[kUT];
  const int b = blockIdx.x, tid = threadIdx.x;
  int32_t* tok = tokens + (long)b * S;
  const float* cf = conf + (long)b * S;
  int n_chosen = 0;
  for (int it = 0; it < n; ++it) {
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    for (int i = lo + tid; i < hi; i += kUT) {
      if (tok[i] != mask_id) continue;
      bool taken = false;
      for (int c = 0; c < n_chosen; ++c) taken |= (chosen[c] == i);
      if (taken) continue;
      const float c = cf[i];
      if (c > best || (c == best && i < bidx)) {
        best = c;
        bidx = i;
      }
    }
    bc[tid] = best;
    bi[tid] = bidx;
    __syncthreads();
    for (int w = kUT / 2; w > 0; w >>= 1) {
      if (tid < w) {
        const float c2 = bc[tid + w];
        const int i2 = bi[tid + w];
        if (c2 > bc[tid] || (c2 == bc[tid] && i2 < bi[tid])) {
          bc[tid] = c2;
          bi[tid] = i2;
        }
      }
      __syncthreads();
    }
    const int pick = bi[0];
    __syncthreads();
    if (pick == 0x7fffffff) break;
    if (tid == 0) chosen[n_chosen] = pick;
    ++n_chosen;
    __syncthreads();
  }
  for (int c = tid; c < n_chosen; c += kUT) tok[chosen[c]] = argmax[(long)b * S + chosen[c]];
}

hipError_t launch_unmask(int32_t* tokens, const float* conf, const int32_t* argmax, int B, int S, int mask_id, int lo,
                         int hi, int n, hipStream_t s) {
  if (B <= 0 || n <= 0 || hi <= lo) return hipSuccess;
  if (n > kMaxUnmask) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_unmask, dim3(B), dim3(kUT), 0, s, tokens, conf, argmax, S, mask_id, lo, hi, n);
  return hipGetLastError();
}

__global__ void k_unmask_forced(int32_t* __restrict__ tokens, const uint8_t* __restrict__ force,
                                const int32_t* __restrict__ argmax, int B, int S, int mask_id, int lo, int hi) {
  const int w = hi - lo;
  const long e = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (e >= (long)B * w) return;
  const int b = (int)(e / w), i = lo + (int)(e - (long)b * w);
  const long p = (long)b * S + i;
  if (tokens[p] == mask_id && force[p] == 1) tokens[p] = argmax[p];
}

hipError_t launch_unmask_forced(int32_t* tokens, const uint8_t* force, const int32_t* argmax, int B, int S,
                                int mask_id, int lo, int hi, hipStream_t s) {
  const long n = (long)B * (hi - lo);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_unmask_forced, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tokens, force, argmax, B, S,
                     mask_id, lo, hi);
  return hipGetLastError();
}

// Dilated unmasking plan (DUS summary, technical summary section 2): round r of a block takes
// the offsets on the stride-a^(R-1-r) grid that the coarser grid of round r-1 (stride a times
// larger) did not already take.  `stride_prev` is 0 for round 0; both strides are clamped to the
// block length, which keeps the membership test unchanged (only offset 0 is a multiple).
__global__ void k_dus_mark(uint8_t* __restrict__ force, int B, int S, int lo, int block, int stride, int stride_prev,
                           uint8_t mark) {
  const long e = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (e >= (long)B * block) return;
  const int b = (int)(e / block), off = (int)(e - (long)b * block);
  const bool in_round = off % stride == 0 && (stride_prev == 0 || off % stride_prev != 0);
  if (!in_round) return;
  uint8_t* f = force + (long)b * S + lo + off;
  if (*f < mark) *f = mark;
}

hipError_t launch_dus_mark(uint8_t* force, int B, int S, int lo, int block, int stride, int stride_prev, uint8_t mark,
                           hipStream_t s) {
  const long n = (long)B * block;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dus_mark, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, force, B, S, lo, block, stride,
                     stride_prev, mark);
  return hipGetLastError();
}

}  // namespace dllm
