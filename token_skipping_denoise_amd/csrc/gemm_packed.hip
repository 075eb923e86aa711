// Active-row products on weights kept in MFMA fragment order (ES-dLLM technical summary 2.1
// item 2: at batch 1 the selected rows make the later layers' products weight-streaming bound,
// M = the active rows).
//
// The weight matrix W [N, K] (nn.Linear layout) is stored a second time, packed so that the B
// operand of one v_mfma_f32_32x32x16_bf16 -- 32 output columns x 16 reduction elements, lane l
// holding columns l % 32 and elements 8 (l / 32) .. +8 -- is one contiguous 1 KB fragment, and
// the four fragments of one 64-element stage of every column block follow each other, stage
// after stage (NB = N / 32 column blocks):
//     fragment (nb, ks) at element ((ks / 4) * NB + nb) * 2048 + (ks % 4) * 512, lane l element e
//         = W[row(32 nb + l % 32)][16 ks + 8 (l / 32) + e].
// All waves of a launch start together, so at any moment they read one contiguous span of the
// packed matrix (stage-major) rather than hundreds of streams a fixed stride apart, which
// measured 15% slower when every launch waits on the one before.
// For the stacked gate/up matrix [gate; up] [2F, K] the packed rows are interleaved in 16s:
// packed row 32 nb + r is gate row 16 nb + r for r < 16 and up row F + 16 nb + r - 16 otherwise,
// so the two factors of one output land in lanes t and t + 16 of the same accumulator.
//
// Each wave owns one 32-column block and all (up to 128) rows: its weight fragments go straight
// from memory into registers, D stages (64 reduction elements each) ahead, one fully coalesced
// 1 KB load per fragment, with no LDS traffic for them; the activation rows, shared by every
// wave, stream through a (D + 1)-stage LDS ring by direct-to-LDS DMA.  The weights are the A
// operand (the product is computed transposed): a lane then holds one activation row and 16 of
// the block's columns, so with the 16-row gate/up interleave the two factors of a feature sit in
// elements e and e + 8 of the same lane, and stores are 8-16 contiguous bytes per lane.  The stage loop is
// unrolled over a compile-time stage count so every wait is exact (a loop back edge makes the
// compiler drain all loads in flight once per trip).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dllm {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPkD = 7;       // weight stages in flight
constexpr int kPkBK = 64;     // reduction elements per stage
constexpr int kPkRows = 128;  // rows per workgroup (the whole active set)

template <int N>
__device__ __forceinline__ void pk_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// at most `ahead` stages of PER loads each still in flight (a constant after unrolling)
template <int MAXA, int PER>
__device__ __forceinline__ void pk_wait_stages(int ahead) {
  if constexpr (MAXA <= 0) {
    pk_wait_vm<0>();
  } else {
    if (ahead >= MAXA) pk_wait_vm<MAXA * PER>();
    else pk_wait_stages<MAXA - 1, PER>(ahead);
  }
}

__device__ __forceinline__ bool rows_live(int M, const int32_t* __restrict__ n_active, int k_max) {
  if (!n_active) return true;
  for (int r = 0; r < M;) {
    const int b = r / k_max, j = r - b * k_max;
    if (j < n_active[b]) return true;
    r = (b + 1) * k_max;
  }
  return false;
}

__global__ void k_pack_frag(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wp, int N, int K, int F) {
  const long nfr = (long)(N / 32) * (K / 16);
  const int l = threadIdx.x & 63;
  for (long f = blockIdx.x * (long)(blockDim.x / 64) + threadIdx.x / 64; f < nfr;
       f += (long)gridDim.x * (blockDim.x / 64)) {
    // f enumerates the packed fragments in memory order: stage kb, column block nb, step s
    const long NB = N / 32;
    const long kb = f / (NB * 4), rem = f - kb * NB * 4, nb = rem >> 2, ks = kb * 4 + (rem & 3);
    const int r = l & 31;
    long src = 32 * nb + r;
    if (F > 0) src = (r < 16) ? 16 * nb + r : F + 16 * nb + (r - 16);
    const uint4 v = *reinterpret_cast<const uint4*>(W + src * K + 16 * ks + 8 * (l >> 5));
    *reinterpret_cast<uint4*>(Wp + f * 512 + l * 8) = v;
  }
}

// Activation tile DMA through a buffer resource over A (a buffer load to LDS issues
// faster than the flat global_load_lds form); word 3 is the raw 32-bit format.
template <int LAW, int NW, int BK>
__device__ __forceinline__ void act_dma(const uint16_t* A, int a_bytes, const int* oa, int k0_bytes, uint16_t* stage,
                                        int wave) {
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, a_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < LAW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(stage + (wave + NW * i) * 8 * BK), 16, oa[i] + k0_bytes, 0,
                                             0, 0);
}

// EPI 0: fp32 split-K partials C[sp][m][n].  EPI 2: H[m][f] = silu(gate) * up (bf16), F outputs.
template <int NW, int NKC, int EPI, int LAW>
__device__ __forceinline__ void packed_body(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Wp,
                                            float* __restrict__ C, uint16_t* __restrict__ H, int M, int N, int K,
                                            int F, int tn, int sp, uint16_t* smem) {
  constexpr int D = kPkD, BK = kPkBK, TM = kPkRows / 32;
  constexpr int PER = LAW + 4;  // loads per stage: LAW activation DMAs + 4 weight fragments
  constexpr int ASTAGE = kPkRows * BK;
  static_assert(NKC >= D, "the prologue fills D stages");
  const int kb0 = sp * NKC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5, r32 = lane & 31;
  // activation DMA: 16 instructions of 8 rows (1 KB) per stage, instruction q = wave + NW i;
  // chunk c of row r sits in slot c ^ ((r >> 1) & 7) so the fragment reads are conflict-free
  // (buffer loads: byte offsets within A, which the launcher keeps under 2^31 bytes)
  int oa[LAW];
#pragma unroll
  for (int i = 0; i < LAW; ++i) {
    const int row = (wave + NW * i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    oa[i] = (min(row, M - 1) * K + chunk * 8) * 2;
  }
  const int a_bytes = M * K * 2;
  const int nb = tn * NW + wave;  // this wave's 32-column block
  const long stage_stride = (long)(N / 32) * 2048;  // one stage of every column block
  const uint16_t* gw = Wp + (long)nb * 2048 + lane * 8;
  bf16x8_t wb[D + 1][4];
  auto issue = [&](int slot, int kb, bf16x8_t* wdst) {
    act_dma<LAW, NW, BK>(A, a_bytes, oa, kb * BK * 2, smem + slot * ASTAGE, wave);
#pragma unroll
    for (int s = 0; s < 4; ++s) wdst[s] = *reinterpret_cast<const bf16x8_t*>(gw + kb * stage_stride + s * 512);
  };
  f32x16_t acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const int swz = (lane >> 1) & 7;
  auto compute = [&](int slot, const bf16x8_t* w) {
    const uint16_t* base = smem + slot * ASTAGE;
    bf16x8_t af[2][TM];
    auto frags = [&](int s, bf16x8_t* dst) {
      const int sl = ((2 * s + hi) ^ swz) * 8;
#pragma unroll
      for (int i = 0; i < TM; ++i) dst[i] = *reinterpret_cast<const bf16x8_t*>(base + (i * 32 + r32) * BK + sl);
    };
    frags(0, af[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) frags(s + 1, af[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // next step's LDS reads stay ahead of this step's MFMAs
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[s], af[s & 1][i], acc[i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) issue(j, kb0 + j, wb[j]);
#pragma unroll
  for (int t = 0; t < NKC; ++t) {
    const int u = t % (D + 1);
    pk_wait_stages<D - 1, PER>(NKC - 1 - t);  // stage t has landed (this wave's loads)
    __builtin_amdgcn_s_barrier();             // ... and every wave's; slot (t - 1) is free
    if (t + D < NKC) issue((u + D) % (D + 1), kb0 + t + D, wb[(u + D) % (D + 1)]);
    compute(u, wb[u]);
  }
  // lane (hi, r32), element e of acc[i]: activation row 32 i + r32, block column
  // 8 (e >> 2) + 4 hi + (e & 3)
  if (EPI == 0) {
    float* Cs = C + (long)sp * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = i * 32 + r32;
      if (row >= M) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(Cs + (long)row * N + nb * 32 + 8 * g + 4 * hi) =
            make_float4(acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]);
    }
  } else {
    // elements e < 8: gate of feature 16 nb + 8 (e >> 2) + 4 hi + (e & 3); e + 8: its up value
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = i * 32 + r32;
      if (row >= M) continue;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t w2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = 4 * g + 2 * h;
          w2[h] = pack_bf16x2(silu_fast(acc[i][e]) * acc[i][e + 8], silu_fast(acc[i][e + 1]) * acc[i][e + 9]);
        }
        *reinterpret_cast<uint2*>(H + (long)row * F + nb * 16 + 8 * g + 4 * hi) = make_uint2(w2[0], w2[1]);
      }
    }
  }
}

template <int NW, int NKC, int EPI>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm_packed(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ Wp, float* __restrict__ C,
                                                            uint16_t* __restrict__ H, int M, int N, int K, int F,
                                                            int tiles_n, const int32_t* __restrict__ n_active,
                                                            int k_max) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(kPkD + 1) * kPkRows * kPkBK];  // 128 KB
  if (!rows_live(M, n_active, k_max)) return;
  const int tn = blockIdx.x % tiles_n, sp = blockIdx.x / tiles_n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // 16 activation DMAs per stage over NW waves: the first 16 % NW waves issue one more
  constexpr int LA_HI = (16 + NW - 1) / NW, LA_LO = 16 / NW;
  if (LA_HI == LA_LO || wave < 16 % NW) packed_body<NW, NKC, EPI, LA_HI>(A, Wp, C, H, M, N, K, F, tn, sp, smem);
  else packed_body<NW, NKC, EPI, LA_LO>(A, Wp, C, H, M, N, K, F, tn, sp, smem);
}

}  // namespace

// Stages per split compiled for each epilogue: the fused gate/up product over d = 4096
// (64 stages), the down projection over F = 12288 in 8 splits (24 stages).
PackedPlan packed_plan(int M, int N, int K, bool swiglu) {
  PackedPlan p;
  if (M < 1 || M > kPkRows || K % kPkBK) return p;
  const int stages = K / kPkBK;
  if (swiglu) {
    // N = 2F packed columns, 96 per workgroup (48 outputs)
    if (N % 96 || stages != 64) return p;
    p.nw = 3;
    p.splits = 1;
  } else {
    if (N % 128) return p;
    const int tiles = N / 128;
    int splits = 1;
    while (tiles * splits < 256 && splits < 8) splits *= 2;
    if (stages % splits || stages / splits != 24) return p;
    p.nw = 4;
    p.splits = splits;
  }
  p.nkc = stages / p.splits;
  p.ok = true;
  return p;
}

hipError_t launch_gemm_packed(const PackedPlan& p, const void* A, const void* Wp, float* C, void* H, int M, int N,
                              int K, int F, const int32_t* n_active, int k_max, hipStream_t s) {
  if (!p.ok || M <= 0 || M > kPkRows || (long)M * K * 2 > 0x7fffffffL) return hipErrorInvalidValue;
  const int tiles_n = N / (32 * p.nw);
  const dim3 grid(tiles_n * p.splits), block(64 * p.nw);
  if (H && p.nw == 3 && p.nkc == 64)
    hipLaunchKernelGGL((k_gemm_packed<3, 64, 2>), grid, block, 0, s, (const uint16_t*)A, (const uint16_t*)Wp, C,
                       (uint16_t*)H, M, N, K, F, tiles_n, n_active, k_max);
  else if (!H && p.nw == 4 && p.nkc == 24)
    hipLaunchKernelGGL((k_gemm_packed<4, 24, 0>), grid, block, 0, s, (const uint16_t*)A, (const uint16_t*)Wp, C,
                       (uint16_t*)H, M, N, K, F, tiles_n, n_active, k_max);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_pack_frag(const void* W, void* Wp, int N, int K, int F, hipStream_t s) {
  const long nfr = (long)(N / 32) * (K / 16);
  if (nfr <= 0) return hipSuccess;
  const long blocks = std::min<long>((nfr + 3) / 4, 65536);
  hipLaunchKernelGGL(k_pack_frag, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t*)W, (uint16_t*)Wp, N, K, F);
  return hipGetLastError();
}

}  // namespace dllm
