// Active-row GEMMs: C[s][m][n] = sum_{k in split s} A[m][k] * W[n][k].
//
// ES-dLLM (technical summary 2.1 item 2) notes that computing only the
// selected rows shrinks the matrix products of the later layers: M becomes
// the number of active rows.  Both operands are K-contiguous (activations
// [M, K], nn.Linear weights [N, K]), which is the natural layout for the
// CDNA matrix cores.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation, WM x WN
// wavefronts (times KG k-groups) per tile, BK = 64, tiles streamed from memory
// straight into a multi-stage LDS ring with 16-byte buffer loads to LDS (no
// register staging), XOR-swizzled so MFMA fragment reads are conflict-free.
// Most plans use eight wavefronts: these kernels are bound by the loads each CU
// keeps in flight, and more waves issue more of them.  Split-K writes fp32
// partials that the row epilogues reduce; row tiles with no live row exit at
// once.
// Workgroup ids are remapped so that each XCD works on a contiguous range of
// tiles, m-tile fastest, so tiles sharing a weight panel share that XCD's L2.
//
// fp32 path (small fp32 models): LDS-tiled FMA kernel, 64x64 tiles.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));


__device__ __forceinline__ bool tile_live(int m0, int bm, int M, const int32_t* __restrict__ n_active, int k_max) {
  if (!n_active) return true;
  const int m1 = min(m0 + bm, M);
  for (int r = m0; r < m1;) {
    const int b = r / k_max, j = r - b * k_max;
    if (j < n_active[b]) return true;
    r = (b + 1) * k_max;
  }
  return false;
}

__device__ __forceinline__ void decode_tile(int nt, int tiles_m, int tiles_n, int& tm, int& tn, int& sp) {
  const int id = blockIdx.x;
  int lin = id;
  if ((nt & 7) == 0) lin = (id & 7) * (nt >> 3) + (id >> 3);
  tm = lin % tiles_m;
  const int rest = lin / tiles_m;
  tn = rest % tiles_n;
  sp = rest / tiles_n;
}

// EPI = 0: store fp32 partials C[sp][m][n].
// EPI = 1: fused SwiGLU.  W is the stacked [gate; up] matrix [2F, K]; the tile
//          covers BN/2 output columns of H = silu(A Wg^T) * (A Wu^T) [M, F]:
//          in each wavefront's half of the tile the first TN/2 column blocks
//          hold gate rows and the last TN/2 the matching up rows, so a lane
//          holds both factors of its outputs.  splits must be 1.
// EPI = 2: fused SwiGLU with gate and up rows interleaved in groups of 16: each 32-row
//          block of the tile holds 16 gate rows and the matching 16 up rows, so the two
//          factors sit in lanes t and t + 16 of one accumulator; any column count that is a
//          multiple of 32 works (48 outputs for 96 columns).
//
// Direct-to-LDS variant (gfx950 buffer_load_dwordx4 ... lds): tiles stream from
// memory straight into an NS-stage LDS ring with no register staging, so
// NS-1 tiles stay in flight while one is multiplied.  BK = 64: a tile row is
// 128 bytes = 8 chunks of 16 bytes; one wave load instruction fills 8 rows
// (1 KB), and chunk c of row r is stored at slot c ^ ((r >> 1) & 7), so the
// MFMA fragment reads (32 rows at one chunk index) are free of bank conflicts.
// s_waitcnt with only vmcnt constrained (expcnt/lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most `ahead` stages of PER loads each are still in flight (ahead <= MAXA).
// An if-chain on a uniform value: a switch would become a jump table (a scalar load and an
// indirect branch on every K step).
template <int MAXA, int PER>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= MAXA) wait_vm<MAXA * PER>();
    else wait_stages<MAXA - 1, PER>(ahead);
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Tile loads go through buffer resources based at the tile's first row, so that
// every offset is a 32-bit byte count within the tile (the launcher checks the
// span) and the address arithmetic is one VGPR add per load.  A buffer load to LDS
// issues faster than the flat global_load_lds form on gfx950.  Word 3 of the
// descriptor is the raw 32-bit-element format with no swizzle.
template <int LA, int LB, int NW, int BM, int BK>
__device__ __forceinline__ void issue_tile(const uint16_t* a_base, int a_bytes, const int* oa, const uint16_t* w_base,
                                           int w_bytes, const int* ob, int k0_bytes, uint16_t* stage, int wave) {
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)w_base, (short)0, w_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < LA; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(stage + (wave + NW * i) * 8 * BK), 16, oa[i] + k0_bytes, 0,
                                             0, 0);
#pragma unroll
  for (int i = 0; i < LB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(stage + BM * BK + (wave + NW * i) * 8 * BK), 16,
                                             ob[i] + k0_bytes, 0, 0, 0);
}

template <int BM, int BN, int NS, int EPI, int OCC, int KG, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN * KG, OCC) void k_gemm_lds(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                     float* __restrict__ C, uint16_t* __restrict__ H, int M, int N,
                                                     int K, int splits, int tiles_m, int tiles_n,
                                                     const int32_t* __restrict__ n_active, int k_max) {
  constexpr int BK = 64;
  constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);  // 32x32 blocks per wave
  constexpr int NW = WM * WN * KG;           // wavefronts
  constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW);  // load instructions per wave per stage (8 rows each)
  constexpr int STAGE = (BM + BN) * BK;      // elements per stage
  constexpr int KS = BK / 16 / KG;           // MFMA k-steps per stage for each k-group
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave tiles are whole 32x32 blocks");
  static_assert(EPI != 1 || TN % 2 == 0, "fused SwiGLU needs an even number of column blocks per wave");
  static_assert(LA * 8 * NW == BM && LB * 8 * NW == BN, "every wave issues the same number of tile loads");
  static_assert(KG == 1 || NS * STAGE * 2 >= BM * BN * 4, "the k-group reduction reuses the stage ring");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE];

  int tmi, tni, sp;
  decode_tile(tiles_m * tiles_n * splits, tiles_m, tiles_n, tmi, tni, sp);
  const int m0 = tmi * BM;
  if (!tile_live(m0, BM, M, n_active, k_max)) return;
  const int nkb = K / BK;
  const int kb0 = (int)((long)sp * nkb / splits), kb1 = (int)((long)(sp + 1) * nkb / splits);
  const int nk = kb1 - kb0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // KG k-groups of WM x WN wavefronts over the tile: group kg multiplies k-steps
  // [kg * KS, (kg + 1) * KS) of every stage; their sums meet in LDS at the end
  const int kg = wave / (WM * WN), w4 = wave % (WM * WN);
  const int wm = w4 / WN, wn = w4 % WN;

  const int F = N;
  const int h0 = tni * (BN / 2);
  // SwiGLU: the tile's columns are WN wave slices of BN / WN; in each slice the first half
  // holds gate rows and the second half the matching up rows
  auto w_row = [&](int c) -> int {
    if (EPI == 0) return tni * BN + c;
    if (EPI == 2) {  // every 32-row block: 16 gate rows, then the 16 matching up rows
      const int o = h0 + (c >> 5) * 16 + (c & 15);
      return (c & 16) ? F + o : o;
    }
    constexpr int SL = BN / WN;
    const int sl = c / SL, lc = c % SL;
    const int jb = lc / 32, t = lc % 32;
    return (jb < TN / 2) ? h0 + sl * (SL / 2) + jb * 32 + t : F + h0 + sl * (SL / 2) + (jb - TN / 2) * 32 + t;
  };
  const int w_rows = (EPI == 0) ? N : 2 * F;
  // A tile row is 128 bytes, half of the 64 banks: rows r and r+1 fall in opposite bank
  // halves, so the chunk slot is swizzled by (r >> 1) & 7 and any 16 consecutive rows read at
  // one chunk index touch all 64 banks once.
  // per-tile bases: A from row m0, W from the tile's lowest weight row (every row the
  // tile reads, clamped rows included, lies at or above it)
  const int wr0 = (EPI == 0) ? tni * BN : h0;
  const uint16_t* a_base = A + (long)m0 * K;
  const uint16_t* w_base = W + (long)wr0 * K;
  const int a_bytes = (int)min((long)(M - m0) * K * 2, 0x7fffffffL);
  const int w_bytes = (int)min((long)(w_rows - wr0) * K * 2, 0x7fffffffL);
  const int lrow = lane >> 3;
  int oa[LA], ob[LB];  // byte offsets of this lane's chunk in each load, k excluded
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = (wave + NW * i) * 8 + lrow;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    oa[i] = ((min(m0 + row, M - 1) - m0) * K + chunk * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int row = (wave + NW * i) * 8 + lrow;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    ob[i] = ((min(w_row(row), w_rows - 1) - wr0) * K + chunk * 8) * 2;
  }
  auto issue = [&](int stage, int kb) {
    issue_tile<LA, LB, NW, BM, BK>(a_base, a_bytes, oa, w_base, w_bytes, ob, kb * BK * 2, smem + stage * STAGE, wave);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int swz = (lane >> 1) & 7, hi = lane >> 5, r32 = lane & 31;  // fragment rows start at multiples of 32
  // fragments of step ks+1 are read from LDS while the MFMAs of step ks run
  auto load_frags = [&](const uint16_t* base, int ks, bf16x8_t* af, bf16x8_t* bfr) {
    const int slot = ((ks * 2 + hi) ^ swz) * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t*>(base + (wm * (BM / WM) + i * 32 + r32) * BK + slot);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(base + BM * BK + (wn * (BN / WN) + j * 32 + r32) * BK + slot);
  };
  auto compute = [&](int stage) {
    const uint16_t* base = smem + stage * STAGE;
    bf16x8_t af[2][TM], bfr[2][TN];
    load_frags(base, kg * KS, af[0], bfr[0]);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int ks = kk;  // buffer parity; the LDS k-step is kg * KS + kk
      if (kk + 1 < KS) load_frags(base, kg * KS + kk + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      // scheduling fence: the next step's LDS reads stay ahead of this step's MFMAs (the
      // scheduler would otherwise sink them behind the MFMAs and stall on their latency)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, kb0 + s);
  for (int t = 0; t < nk; ++t) {
    wait_stages<NS - 2, LA + LB>(nk - 1 - t);  // tiles after t may stay in flight
    // barrier without a memory fence: a fence would wait for every load in flight
    __builtin_amdgcn_s_barrier();
    if (t + NS - 1 < nk) issue((t + NS - 1) % NS, kb0 + t + NS - 1);
    compute(t % NS);
  }
  if constexpr (KG == 2) {
    // k-group 1 hands its sums to k-group 0 through the (now idle) stage ring
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) red[(((w4 * TM + i) * TN + j) * 16 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += red[(((w4 * TM + i) * TN + j) * 16 + e) * 64 + lane];
  }

  if (EPI == 0) {
    float* Cs = C + (long)sp * M * N;
    const int n0 = tni * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row < M) Cs[(long)row * N + col] = acc[i][j][e];
        }
      }
  } else if (EPI == 2) {
    // lane t < 16 of a column block holds gate output t, lane t + 16 the matching up value
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = h0 + ((wn * (BN / WN) + j * 32) >> 1) + (lane & 15);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = acc[i][j][e];
          const float u = __shfl_xor(v, 16, kWave);
          const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if ((lane & 16) == 0 && col < F && row < M) H[(long)row * F + col] = f2bf(silu_fast(v) * u);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int col = h0 + wn * (BN / WN / 2) + j * 32 + (lane & 31);
        if (col >= F) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row >= M) continue;
          const float g = acc[i][j][e], u = acc[i][j + TN / 2][e];
          H[(long)row * F + col] = f2bf(silu_fast(g) * u);
        }
      }
  }
}

// fp32: 64x64 tile, BK 16, 256 threads x (4x4) outputs.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, const float* __restrict__ W,
                                                  float* __restrict__ C, int M, int N, int K, int splits, int tiles_m,
                                                  int tiles_n, const int32_t* __restrict__ n_active, int k_max) {
  __shared__ float As[16][64 + 4], Ws[16][64 + 4];
  int tmi, tni, sp;
  decode_tile(tiles_m * tiles_n * splits, tiles_m, tiles_n, tmi, tni, sp);
  const int m0 = tmi * 64, n0 = tni * 64;
  if (!tile_live(m0, 64, M, n_active, k_max)) return;
  const int nkb = (K + 15) / 16;
  const int kb0 = (int)((long)sp * nkb / splits), kb1 = (int)((long)(sp + 1) * nkb / splits);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int kb = kb0; kb < kb1; ++kb) {
    const int k0 = kb * 16;
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e >> 4, kk = e & 15;
      const int gk = k0 + kk;
      As[kk][r] = (m0 + r < M && gk < K) ? A[(long)(m0 + r) * K + gk] : 0.f;
      Ws[kk][r] = (n0 + r < N && gk < K) ? W[(long)(n0 + r) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Cs = C + (long)sp * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < M && col < N) Cs[(long)row * N + col] = acc[i][j];
    }
}

#ifndef DLLM_LDS_CASES
#define DLLM_LDS_CASES                                                                              \
  DLLM_LDS_CASE(128, 64, 4, 1, 2, 2) DLLM_LDS_CASE(128, 128, 2, 1, 2, 2) DLLM_LDS_CASE(128, 128, 3, 1, 2, 2) \
  DLLM_LDS_CASE(128, 256, 3, 1, 2, 4) DLLM_LDS_CASE(256, 256, 2, 1, 2, 4) DLLM_LDS_CASE(128, 128, 4, 2, 2, 2) \
  DLLM_LDS_CASE(256, 192, 2, 1, 4, 2) DLLM_LDS_CASE(256, 128, 3, 1, 4, 2) DLLM_LDS_CASE(128, 192, 3, 1, 4, 2) \
  DLLM_LDS_CASE(128, 64, 4, 1, 4, 2) DLLM_LDS_CASE(128, 128, 3, 1, 4, 2)
#endif
#ifndef DLLM_LDS_SWIGLU_CASES
#define DLLM_LDS_SWIGLU_CASES                                                                       \
  DLLM_LDS_CASE(128, 128, 3, 1, 2, 2) DLLM_LDS_CASE(128, 128, 3, 2, 2, 2)
#endif

#ifndef DLLM_LDS_SWIGLU_ILV_CASES
#define DLLM_LDS_SWIGLU_ILV_CASES \
  DLLM_LDS_CASE(128, 96, 4, 1, 4, 1) DLLM_LDS_CASE(256, 192, 2, 1, 4, 2) DLLM_LDS_CASE(128, 256, 2, 1, 2, 4)
#endif

GemmPlan gemm_plan(int dtype, int M, int N, int K, bool swiglu) {
  GemmPlan p{64, 64, 1, 64, 2};
  if (dtype == 0) {
    const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
    while (!swiglu && tiles * p.splits < 256 && p.splits < 8 && (K / 16) / (p.splits * 2) >= 8) p.splits *= 2;
    return p;
  }
  // Direct-to-LDS kernel (pd = 10 + stages).  Rules from tile sweeps on the LLaDA-8B layer
  // shapes.  Few rows (HBM bound on the weights): 128-row tiles over eight wavefronts (more
  // waves issuing loads keep more bytes in flight per CU); wide QKV-like outputs take 192
  // columns (256 over 2 x 4 when 192 does not divide them), narrow ones 64 columns with 4
  // stages, and split-K fills the chip.  Many rows: 256-row tiles over 4 x 2 wavefronts where
  // the shape allows (256 x 192 for the fused SwiGLU product and QKV-like outputs, 256 x 128
  // with a 4- or 2-way K split for the down projection), otherwise 128 x 128 with 2 stages, so
  // that two workgroups share a CU, and split-K up to 4.  With rows padded per sequence, dead
  // rows fill more of a 256-row tile than of a 128-row one: a SwiGLU width that 96 does not
  // divide takes interleaved 128 x 256 tiles (faster at every live share measured on
  // Dream-7B's F = 18944 than 256 x 128 ones, which win only on fully live rows).
  const bool few = M <= 192;
  const bool wide = N > 8192 && N <= 32768;
  p.bm = 128;
  p.bn = 128;
  long target = 256;
  if (few) {
    if (swiglu) {
      // the fused epilogue needs whole sums, so no split-K: 48 outputs per tile (gate and up
      // rows interleaved in 16s) give enough tiles to fill the chip when they divide F
      if (N % 48 == 0 && N / 48 >= 192) {
        p.bn = 96;
        p.wm = 4;
        p.wn = 1;
        p.pd = 14;
        p.ilv = 1;
      } else {
        p.pd = 13;
      }
      return p;
    }
    if (wide) {
      // 128 x 192 tiles over 4 x 2 wavefronts when they divide the width: 4-way split-K then
      // gives 256 workgroups, one per CU
      p.bn = (N % 192 == 0) ? 192 : 256;
      p.wm = (p.bn == 192) ? 4 : 2;
      p.wn = (p.bn == 192) ? 2 : 4;
      p.pd = 13;
      target = 192;
    } else if (N > 32768) {
      p.wm = 4;
      p.pd = 13;
    } else if (K >= 2 * N && K % (8 * 64 * 4) == 0 && N % 128 == 0) {
      // long reductions into narrow outputs (the down projection): 128 x 128 tiles with two
      // k-groups of wavefronts (two waves per SIMD) and an 8-way K split to fill the chip
      p.pd = 14;
      p.kg = 2;
      p.splits = 8;
      return p;
    } else {
      p.bn = 64;
      p.wm = 4;
      p.pd = 14;
    }
  } else {
    // 256-row tiles over 4 x 2 wavefronts: 64 x 96 (or 64 x 64) wave tiles, and eight waves
    // issuing the tile loads (the loads in flight per CU, not the MFMAs, bound these tiles)
    if (swiglu) {
      if (N % 96 == 0) {  // 96 outputs (192 interleaved gate/up rows) per tile
        p.bm = 256;
        p.bn = 192;
        p.wm = 4;
        p.wn = 2;
        p.pd = 12;
        p.ilv = 1;
      } else if (N % 128 == 0) {  // 128 outputs over 128-row tiles (Dream-7B's F = 18944)
        p.bn = 256;
        p.wm = 2;
        p.wn = 4;
        p.pd = 12;
        p.ilv = 1;
      } else {
        p.pd = 13;
        p.kg = 2;
      }
      return p;
    }
    if (wide) {
      p.bm = 256;
      p.bn = (N % 192 == 0) ? 192 : 256;
      p.wm = (p.bn == 192) ? 4 : 2;
      p.wn = (p.bn == 192) ? 2 : 4;
      p.pd = 12;
      target = 192;
    } else if (K >= 2 * N && N % 128 == 0 && K / (64 * 4) >= 3) {
      // long reductions into narrow outputs (the down projection): a 4-way K split, 2-way
      // once the row tiles alone give three workgroups per CU
      p.bm = 256;
      p.wm = 4;
      p.wn = 2;
      p.pd = 13;
      p.splits = ((long)((M + 255) / 256) * ((N + 127) / 128) >= 768) ? 2 : 4;
      return p;
    } else if (N % 192 == 0 && N <= 32768) {
      // QKV-like widths below the wide range (Dream-7B's 4608): 128 x 192 over 4 x 2 waves,
      // measured no slower than 128 x 128 at any live share and 15% faster on live rows
      p.bn = 192;
      p.wm = 4;
      p.wn = 2;
      p.pd = 13;
    } else {
      p.pd = 12;
      target = 512;
    }
  }
  const long tiles = (long)((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  const int max_splits = 4;
  while (tiles * p.splits < target && p.splits < max_splits && K / (p.splits * 2) >= 1024) p.splits *= 2;
  return p;
}

template <int BM, int BN, int NS, int EPI, int KG, int WM, int WN>
static hipError_t launch_lds(const GemmPlan& p, const void* A, const void* W, float* C, void* H, int M, int N, int K,
                             const int32_t* n_active, int k_max, hipStream_t s) {
  // the kernel's buffer offsets are 32-bit bytes within one tile: BM rows of A, and
  // BN weight rows (plain) or the gate..up span F + BN / 2 rows (SwiGLU)
  const long w_span = EPI == 0 ? BN : (long)N + BN / 2;
  if ((long)BM * K * 2 > 0x7fffffffL || w_span * K * 2 > 0x7fffffffL) return hipErrorInvalidValue;
  const int ncols = EPI == 0 ? BN : BN / 2;
  const int tm = (M + BM - 1) / BM, tn = (N + ncols - 1) / ncols;
  constexpr int lds_bytes = NS * (BM + BN) * 64 * 2;
  constexpr int occ = (lds_bytes <= 80 * 1024 && KG * WM * WN == 4) ? 2 : 1;
  hipLaunchKernelGGL((k_gemm_lds<BM, BN, NS, EPI, occ, KG, WM, WN>), dim3(tm * tn * p.splits), dim3(64 * KG * WM * WN), 0, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, (uint16_t*)H, M, N, K, p.splits, tm, tn, n_active, k_max);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, const GemmPlan& p, const void* A, const void* W, float* C, int M, int N, int K,
                       const int32_t* n_active, int k_max, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 0) {
    const int tm = (M + 63) / 64, tn = (N + 63) / 64;
    hipLaunchKernelGGL(k_gemm_f32, dim3(tm * tn * p.splits), dim3(256), 0, s, (const float*)A, (const float*)W, C, M,
                       N, K, p.splits, tm, tn, n_active, k_max);
    return hipGetLastError();
  }
  if (K % 64 != 0) return hipErrorInvalidValue;
#define DLLM_LDS_CASE(BM_, BN_, NS_, KG_, WM_, WN_)                                                \
  if (p.bm == BM_ && p.bn == BN_ && p.bk == 64 && p.pd == 10 + NS_ && p.kg == KG_ && p.wm == WM_ &&  \
      p.wn == WN_) {                                                                                \
    return launch_lds<BM_, BN_, NS_, 0, KG_, WM_, WN_>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s); \
  }
  DLLM_LDS_CASES
#undef DLLM_LDS_CASE
#undef DLLM_GEMM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_swiglu(const GemmPlan& p, const void* A, const void* W_gate_up, void* H, int M, int F, int K,
                              const int32_t* n_active, int k_max, hipStream_t s) {
  if (M <= 0 || F <= 0) return hipSuccess;
  if (K % 64 != 0 || F % (p.bn / 2) != 0 || p.splits != 1) return hipErrorInvalidValue;
#define DLLM_LDS_CASE(BM_, BN_, NS_, KG_, WM_, WN_)                                                \
  if (p.bm == BM_ && p.bn == BN_ && p.bk == 64 && p.pd == 10 + NS_ && p.kg == KG_ && p.wm == WM_ &&  \
      p.wn == WN_ && !p.ilv) {                                                                      \
    return launch_lds<BM_, BN_, NS_, 1, KG_, WM_, WN_>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s); \
  }
  DLLM_LDS_SWIGLU_CASES
#undef DLLM_LDS_CASE
#define DLLM_LDS_CASE(BM_, BN_, NS_, KG_, WM_, WN_)                                                \
  if (p.bm == BM_ && p.bn == BN_ && p.bk == 64 && p.pd == 10 + NS_ && p.kg == KG_ && p.wm == WM_ &&  \
      p.wn == WN_ && p.ilv) {                                                                       \
    return launch_lds<BM_, BN_, NS_, 2, KG_, WM_, WN_>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s); \
  }
  DLLM_LDS_SWIGLU_ILV_CASES
#undef DLLM_LDS_CASE
#undef DLLM_SWIGLU_CASE
  return hipErrorInvalidValue;
}

}  // namespace dllm
