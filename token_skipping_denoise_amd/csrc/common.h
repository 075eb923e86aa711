// Internal helpers shared by the gfx950 kernels of libdllm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

constexpr int kWave = 64;  // CDNA wavefront width

// ---- bf16 storage (raw 16-bit patterns; arithmetic is always fp32) ----
struct bf16 {
  uint16_t v;
};

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// silu(x) = x / (1 + e^-x) on the hardware exp2 and reciprocal (a few 1e-7 relative error;
// the limits 0 and x come out exactly for large |x|)
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bf16 in one instruction (v_cvt_pk_bf16_f32: round to nearest even, NaN
// stays NaN), a in the low half.  A bit-twiddling rounding with its NaN test costs a branch
// per element, which made output conversion a visible part of short kernels.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ float ld(const float* p, long i) { return p[i]; }
  __device__ static __forceinline__ void st(float* p, long i, float v) { p[i] = v; }
  // 16-byte chunk <-> fp32 lanes
  __device__ static __forceinline__ void unpack(const uint4& c, float* f) {
    f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};
template <> struct Elem<bf16> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ float ld(const bf16* p, long i) { return bf2f(p[i].v); }
  __device__ static __forceinline__ void st(bf16* p, long i, float v) { p[i].v = f2bf(v); }
  __device__ static __forceinline__ void unpack(const uint4& c, float* f) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// ---- wave reductions (fixed butterfly order: deterministic) ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// Precondition checks of the debug build (compiled with -DDLLM_CHECK): a violated precondition
// sets its bit in a device error word, while the kernel still keeps every access in bounds (the
// row is treated as dead, the token id clamped).  The normal build compiles the checks out.
enum { kChkActiveCount = 1, kChkIndexRange = 2, kChkIndexOrder = 4, kChkTokenRange = 8 };
__device__ __forceinline__ void check_flag(uint32_t* word, uint32_t bit) {
#ifdef DLLM_CHECK
  if (word) atomicOr(word, bit);
#else
  (void)word;
  (void)bit;
#endif
}

// Flat position of an active row in the padded layout, or -1 if the row is dead.
__device__ __forceinline__ int row_position(const int32_t* idx, const int32_t* n_active, int k_max, int S, int r) {
  const int b = r / k_max, j = r - b * k_max;
  if (j >= n_active[b]) return -1;
  return b * S + idx[r];
}

}  // namespace dllm
