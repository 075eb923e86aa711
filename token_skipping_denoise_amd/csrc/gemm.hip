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
// Plans use eight to sixteen wavefronts: these kernels are bound by the loads each
// CU keeps in flight, and more waves issue more of them (LDS reads are not the
// limit); when a tile's load instructions do not divide over all its waves, only
// the first NL of them load.  Split-K writes fp32 partials that the row epilogues
// reduce; row tiles with no live row exit at once.
// Workgroup ids are remapped so that each XCD works on a contiguous range of
// tiles, walked in groups of four row tiles, so the workgroups running together
// on an XCD share both operands' k-slabs through its L2.
//
// Register-staged variant (k_gemm_vr, the 256-row plans from 512 rows on, 256 x 256
// tiles from thousands of rows on): four wavefronts, one per SIMD, stage the tiles through two
// register sets two K stages ahead into a two-slot LDS ring, with every other
// instruction placed between two MFMAs; same layout, k order and results.
//
// fp32 path (small fp32 models): LDS-tiled FMA kernel, 64x64 tiles.
#include <type_traits>

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

// Tile order.  Workgroups are dealt to the eight XCDs in turn by linear id; when the grid is a
// multiple of 8, XCD x takes the x-th contiguous eighth of the tile list instead.  Within a split
// the list runs over groups of kGroupM row tiles: the workgroups running together on one XCD
// cover kGroupM row tiles x several column tiles, so both operands' current k-slabs are shared
// through that XCD's L2 (row tiles fastest over all rows would share only the weights).  With at
// most kGroupM row tiles this is the plain row-fastest order.  On one Dream-7B layer over 8192
// rows, groups of 4 against row-fastest: gate/up 2110 -> 2030 us, QKV + down 773 -> 728 us on
// average, O 302 -> 240 us (groups of 1: 2097 / 776 / 244; of 8: 2041 / 736 / 258).
constexpr int kGroupM = 4;
__device__ __forceinline__ void decode_tile(int nt, int tiles_m, int tiles_n, int& tm, int& tn, int& sp) {
  const int id = blockIdx.x;
  int lin = id;
  if ((nt & 7) == 0) lin = (id & 7) * (nt >> 3) + (id >> 3);
  const int per_split = tiles_m * tiles_n;
  sp = lin / per_split;
  lin -= sp * per_split;
  const int g0 = (lin / (kGroupM * tiles_n)) * kGroupM;
  const int gm = min(kGroupM, tiles_m - g0);
  const int r = lin - g0 * tiles_n;
  tm = g0 + r % gm;
  tn = r / gm;
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

template <int BM, int BN, int NS, int EPI, int OCC, int KG, int WM, int WN, int NL>
__global__ __launch_bounds__(64 * WM * WN * KG, OCC) void k_gemm_lds(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                     float* __restrict__ C, uint16_t* __restrict__ H, int M, int N,
                                                     int K, int splits, int tiles_m, int tiles_n,
                                                     const int32_t* __restrict__ n_active, int k_max) {
  constexpr int BK = 64;
  constexpr int TM = BM / (32 * WM), TN = BN / (32 * WN);  // 32x32 blocks per wave
  constexpr int NW = WM * WN * KG;           // wavefronts
  // the first NL waves issue the tile loads (NL = 0: all of them)
  constexpr int NLW = NL > 0 ? NL : NW;
  constexpr int LA = BM / (8 * NLW), LB = BN / (8 * NLW);  // load instructions per loading wave per stage (8 rows each)
  constexpr int STAGE = (BM + BN) * BK;      // elements per stage
  constexpr int KS = BK / 16 / KG;           // MFMA k-steps per stage for each k-group
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave tiles are whole 32x32 blocks");
  static_assert(EPI != 1 || TN % 2 == 0, "fused SwiGLU needs an even number of column blocks per wave");
  static_assert(LA * 8 * NLW == BM && LB * 8 * NLW == BN && NLW <= NW, "every loading wave issues the same loads");
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
    const int row = (wave + NLW * i) * 8 + lrow;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    oa[i] = ((min(m0 + row, M - 1) - m0) * K + chunk * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int row = (wave + NLW * i) * 8 + lrow;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    ob[i] = ((min(w_row(row), w_rows - 1) - wr0) * K + chunk * 8) * 2;
  }
  const bool loads = NL == 0 || wave < NL;
  auto issue = [&](int stage, int kb) {
    if (loads)
      issue_tile<LA, LB, NLW, BM, BK>(a_base, a_bytes, oa, w_base, w_bytes, ob, kb * BK * 2, smem + stage * STAGE,
                                       wave);
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
    if (loads) wait_stages<NS - 2, LA + LB>(nk - 1 - t);  // tiles after t may stay in flight
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

// Register-staged: 256 x BN tiles (BN = 256, 192 or 128) over four wavefronts (2 x 2, one per
// SIMD, 128 x BN/2 wave tiles whose accumulators, up to 256 per lane, sit in the AGPRs).  The
// direct-to-LDS kernel above keeps one 64-element K stage in flight beside the one being
// multiplied (two 64 KB stages fill most of the LDS); here the stage loads go to registers first,
// in two register sets (each wave loads a quarter of a stage: 8 rows of A and BN / 32 of W, 16 B
// per lane each), so two stages (up to 128 KB per CU) are in flight while one is multiplied from
// a two-slot LDS ring.  With one wave per SIMD nothing else covers a wave's own waits, so every
// k-step issues its 4 x BN / 64 MFMAs one at a time with the other work between them: the LDS
// fragment reads of the next k-step, a third of the LDS writes of the next stage's register set
// and the loads that refill the written registers with the stage after it.  The LDS layout,
// fragment reads, k order and epilogues (EPI 0: fp32 partials; EPI 2: SwiGLU over gate/up rows
// interleaved in 16s) are those of k_gemm_lds, so both kernels give bit-identical results.
// Measured against the direct-to-LDS kernels on the same inputs, launches alternated, median of
// 25.  256 x 256 against 16 waves: Dream-7B at 8192 rows down (2 splits) 992 -> 928 us and O
// 226 -> 212 us (against its 128 x 128 plan); LLaDA-8B at 16384 rows QKV 1360 -> 1294, O
// 492 -> 453, down 1372 -> 1318 us and the LM head 13.89 -> 13.21 ms; the fused SwiGLU product
// the same either way alone (1810 against 1817 us at 8192 rows) but faster inside whole runs; at
// 512 and 820 rows these tiles leave too many CUs idle and are slower.  256 x 192 against 12
// waves: QKV 57.2 -> 55.0 us at 512 rows, 105.7 -> 100.9 at 820, 282.5 -> 269.6 at 8192
// (Dream-7B); gate/up + SwiGLU 115.5 -> 111.4 at 512, 213.1 -> 210.7 at 820.  256 x 128 against
// 16 waves: the split-K down product 60.4 -> 56.7 us at 512 rows, 122.8 -> 116.6 at 820.
template <int EPI, int BN>
__global__ __launch_bounds__(256, 1) void k_gemm_vr(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                    float* __restrict__ C, uint16_t* __restrict__ H, int M, int N, int K,
                                                    int splits, int tiles_m, int tiles_n,
                                                    const int32_t* __restrict__ n_active, int k_max) {
  constexpr int BM = 256, BK = 64, TM = 4, TN = BN / 64;
  constexpr int NB = BN / 32;  // W chunks per lane and stage
  constexpr int NQ = 8 + NB;   // chunks per register set
  constexpr int NF = 4 + TN;   // fragments per k-step
  constexpr int NM = TM * TN;  // MFMAs per k-step
  static_assert(BN == 256 || BN == 192 || BN == 128, "256-, 192- or 128-column tiles");
  constexpr int STAGE = (BM + BN) * BK;  // elements per ring slot
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];  // 96-128 KB

  int tmi, tni, sp;
  decode_tile(tiles_m * tiles_n * splits, tiles_m, tiles_n, tmi, tni, sp);
  const int m0 = tmi * BM;
  if (!tile_live(m0, BM, M, n_active, k_max)) return;
  const int nkb = K / BK;
  const int kb0 = (int)((long)sp * nkb / splits), kb1 = (int)((long)(sp + 1) * nkb / splits);
  const int nk = kb1 - kb0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int F = N;  // SwiGLU: N is the number of outputs F; W holds 2F rows
  const int h0 = tni * (BN / 2);
  const int w_rows = (EPI == 0) ? N : 2 * F;
  const int wr0 = (EPI == 0) ? tni * BN : h0;
  // The last row tile is moved up to end at row M (the launcher ensures M >= 256): it multiplies
  // rows a0 .. a0 + 255 and stores only those from m0 on, so every load stays inside A.  Weight
  // rows never pass the end (N a multiple of BN, or F of BN / 2 for SwiGLU).
  const int a0 = min(m0, M - BM);
  const uint16_t* a_base = A + (long)a0 * K;
  const uint16_t* w_base = W + (long)wr0 * K;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, BM * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)w_base, (short)0, (int)min((long)(w_rows - wr0) * K * 2, 0x7fffffffL), 0x00020000);
  // this lane's loads: chunk c of A rows rb + 32 i (i < 8) and of NB weight rows.  The lane's part
  // of the byte offset is one VGPR per operand; the row step and k go in the scalar offset.
  const int c = tid & 7, rb = tid >> 3;
  // weight row of tile row rb + 32 i: wb0 + i * wstep (SwiGLU: 16 gate rows, then the 16 matching
  // up rows, per 32-row block)
  const int wb0 = (EPI == 0) ? tni * BN + rb : ((rb & 16) ? F : 0) + h0 + (rb & 15);
  constexpr int wstep = (EPI == 0) ? 32 : 16;
  const int va = (rb * K + c * 8) * 2, vw = ((wb0 - wr0) * K + c * 8) * 2;
  // LDS byte address of this lane's chunk in row rb of a slot; rows rb + 32 i share the swizzle
  const uint32_t wr_lds = (uint32_t)(rb * BK * 2 + ((c ^ ((rb >> 1) & 7)) << 4));

  u32x4_t R0[NQ], R1[NQ];  // register sets: stage s lives in set s & 1 (8 A chunks, then NB W chunks)
  // chunk q of a set: A rows rb + 32 q (q < 8), W rows wb0 + wstep (q - 8)
  auto load_one = [&](u32x4_t* R, int q, int kb) {
    const int kbytes = kb * BK * 2;
    if (q < 8) R[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, q * 32 * K * 2 + kbytes, 0);
    else R[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw, (q - 8) * wstep * K * 2 + kbytes, 0);
  };
  auto write_one = [&](const u32x4_t* R, int q, int slot) {
    uint8_t* base = reinterpret_cast<uint8_t*>(smem + slot * STAGE) + wr_lds;
    const int row = (q < 8) ? q * 32 : BM + (q - 8) * 32;
    *reinterpret_cast<u32x4_t*>(base + row * BK * 2) = R[q];
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int swz = (lane >> 1) & 7, hi = lane >> 5, r32 = lane & 31;
  // fragment f < 4: A row block f; f >= 4: W column block f - 4
  auto frag_addr = [&](const uint16_t* base, int ks, int f) {
    const int slot = ((ks * 2 + hi) ^ swz) * 8;
    return (f < 4) ? base + (wm * (BM / 2) + f * 32 + r32) * BK + slot
                   : base + BM * BK + (wn * (BN / 2) + (f - 4) * 32 + r32) * BK + slot;
  };
  bf16x8_t fr[2][NF];  // k-step fragments, double-buffered: k-step ks of a stage in fr[ks & 1]
  // Iteration t multiplies stage t (slot t & 1).  During its first three k-steps it writes stage
  // t + 1 from set Rn into slot (t + 1) & 1 -- last read before the barrier of iteration t - 1 --
  // chunk by chunk, refilling each written register with stage t + 3 right after.  Loads complete
  // in order, and before the write of chunk q exactly 2 NQ - 1 of this wave's loads were issued
  // after the one it needs (Rn's chunks after q, the other set's NQ and the q refills made
  // since), so every wait is vmcnt(2 NQ - 1).  The barrier comes before the last k-step: by then every wave's
  // writes of stage t + 1 have landed and its reads of slot t & 1 are done (the last k-step's
  // fragments were read during the one before), so the last k-step's MFMAs cover the reads of
  // stage t + 1's first fragments.  Past the last stage the refill reads the last stage again and
  // the writes fill a slot nothing multiplies any more, so every iteration is the same code.
  auto iteration = [&](int t, u32x4_t* Rn) {
    const uint16_t* base = smem + (t & 1) * STAGE;
    const uint16_t* nbase = smem + ((t + 1) & 1) * STAGE;
    const int kb_refill = kb0 + min(t + 3, nk - 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks == BK / 16 - 1) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      // chunks written in this k-step: a third of the set in each of the first three
      const int q0 = (ks * NQ + 2) / 3, q1 = ((ks + 1) * NQ + 2) / 3;
      const int nq = (ks < 3) ? q1 - q0 : 0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int i = m / TN, j = m % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks & 1][i], fr[ks & 1][4 + j], acc[i][j], 0, 0, 0);
        // fragment f of the next k-step (the next stage's first after the last) after MFMA 2 f,
        // or after the last MFMA for the fragments the even slots do not reach
        const int f = ((m & 1) == 0) ? (m >> 1) : (m == NM - 1 ? NM / 2 : NF);
        if (f < NF) {
#pragma unroll
          for (int g = f; g < ((m == NM - 1) ? NF : f + 1); ++g) {
            if (ks + 1 < BK / 16)
              fr[(ks + 1) & 1][g] = *reinterpret_cast<const bf16x8_t*>(frag_addr(base, ks + 1, g));
            else
              fr[0][g] = *reinterpret_cast<const bf16x8_t*>(frag_addr(nbase, 0, g));
          }
        }
        if ((m & 1) == 1 && (m >> 1) < nq) {  // one chunk written, then its register refilled
          const int q = q0 + (m >> 1);
          wait_vm<2 * NQ - 1>();
          write_one(Rn, q, (t + 1) & 1);
          load_one(Rn, q, kb_refill);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // prologue (nk >= 3, the launcher's condition): stages 0 and 1 in flight, stage 0 into slot 0,
  // stage 2 into the freed set, then stage 0's first fragments
#pragma unroll
  for (int q = 0; q < NQ; ++q) load_one(R0, q, kb0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) load_one(R1, q, kb0 + 1);
  wait_vm<NQ>();
#pragma unroll
  for (int q = 0; q < NQ; ++q) write_one(R0, q, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) load_one(R0, q, kb0 + 2);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int f = 0; f < NF; ++f) fr[0][f] = *reinterpret_cast<const bf16x8_t*>(frag_addr(smem, 0, f));
  int t = 0;
  for (; t + 1 < nk; t += 2) {  // stage t + 1 is in set 1, stage t + 2 in set 0
    iteration(t, R1);
    iteration(t + 1, R0);
  }
  if (t < nk) iteration(t, R1);  // an odd stage count: the last stage
  wait_vm<0>();                   // no load is left in flight at the end
  __builtin_amdgcn_s_waitcnt(0xc07f);

  if (EPI == 0) {
    float* Cs = C + (long)sp * M * N;
    const int n0 = tni * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * (BN / 2) + j * 32 + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = a0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          if (row >= m0) Cs[(long)row * N + col] = acc[i][j][e];
        }
      }
  } else {
    // lane t < 16 of a column block holds gate output t, lane t + 16 the matching up value
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = h0 + ((wn * (BN / 2) + j * 32) >> 1) + (lane & 15);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = acc[i][j][e];
          const float u = __shfl_xor(v, 16, kWave);
          const int row = a0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          if ((lane & 16) == 0 && row >= m0) H[(long)row * F + col] = f2bf(silu_fast(v) * u);
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

#define DLLM_LDS_CASES                                                                              \
  DLLM_LDS_CASE(128, 64, 4, 1, 2, 2) DLLM_LDS_CASE(128, 128, 2, 1, 2, 2) DLLM_LDS_CASE(128, 128, 3, 1, 2, 2) \
  DLLM_LDS_CASE(128, 256, 3, 1, 2, 4) DLLM_LDS_CASE(256, 256, 2, 1, 2, 4) DLLM_LDS_CASE(128, 128, 4, 2, 2, 2) \
  DLLM_LDS_CASE(128, 192, 3, 1, 4, 2) \
  DLLM_LDS_CASE(128, 64, 4, 1, 4, 2) DLLM_LDS_CASE(128, 128, 3, 1, 4, 2) DLLM_LDS_CASE(256, 256, 2, 1, 4, 4) \
  DLLM_LDS_CASE(256, 128, 3, 1, 4, 4)
#define DLLM_LDS_SWIGLU_CASES                                                                       \
  DLLM_LDS_CASE(128, 128, 3, 1, 2, 2) DLLM_LDS_CASE(128, 128, 3, 2, 2, 2)

#define DLLM_LDS_SWIGLU_ILV_CASES \
  DLLM_LDS_CASE(128, 96, 4, 1, 4, 1) DLLM_LDS_CASE(128, 256, 2, 1, 2, 4) \
  DLLM_LDS_CASE(256, 256, 2, 1, 4, 4)

// Thousands of rows (the Dream-7B steps over 8 x 1024 positions, the long-context refreshes over
// 4 x 4096): 256 x 256 tiles over sixteen wavefronts (4 x 4, four per SIMD, 64 x 64 wave tiles)
// once the launch holds at least this many workgroups.  At 8192 rows of the Dream-7B layer they
// took gate/up + SwiGLU 2697 -> 2046 us, down 1319-1370 -> 1168 us and QKV + down together
// 1678 -> 1478-1485 us against the 8-wave plans below (the lock-ramp run 283 -> 312 tokens/s,
// the long-context run 417 -> 452);
// at 512 and 820 rows, with one or two such workgroups per CU, they were slower (gate/up 102.7
// against 112.4 and 216.7 against 233.5 us), so those keep their tiles.
constexpr long kWideTileWgsSwiglu = 1024;  // four per CU
// The register-staged kernel (k_gemm_vr) from this many rows on: at 512 and 820 rows, with a few
// hundred such workgroups, it measured slower than the direct-to-LDS plans (QKV 113.4 against
// 101.4 us at 820 rows, launches alternated).
constexpr int kVrRows = 2048;
constexpr long kWideTileWgs = 512;         // two per CU
// share of the CU slots that a launch of `wgs` one-per-CU workgroups keeps busy over its rounds
static double round_fill(long wgs) {
  const long cus = 256;
  return (double)wgs / (double)(((wgs + cus - 1) / cus) * cus);
}
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
  // stages, and split-K fills the chip.  Thousands of rows: 256 x 256 tiles over 4 x 4
  // wavefronts when they fill the CUs two (four for SwiGLU) times over.  Many rows: 256-row
  // tiles where the shape allows (256 x 192 over 4 x 3 wavefronts, 8 of them loading, for the
  // fused SwiGLU product and QKV-like outputs: 6-9% faster than over 4 x 2 at 512 and 820
  // rows; 256 x 128 over 4 x 4 with a 4- or 2-way K split for the down projection), otherwise
  // 128 x 128 with 2 stages, so that two workgroups share a CU, and split-K up to 4.  With rows
  // padded per sequence, dead rows fill more of a 256-row tile than of a 128-row one: a SwiGLU
  // width that 96 does not divide takes interleaved 128 x 256 tiles (faster at every live share
  // measured on Dream-7B's F = 18944 than 256 x 128 ones, which win only on fully live rows).
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
    // 256-row tiles with 64 x 64 (or 64 x 96 for the down projection's 256 x 128) wave tiles,
    // eight or more waves issuing the tile loads (the loads in flight per CU, not the MFMAs,
    // bound these tiles)
    if (swiglu) {
      if (N % 128 == 0 && (long)((M + 255) / 256) * (N / 128) >= kWideTileWgsSwiglu) {
        // 128 outputs (256 interleaved gate/up rows) per tile; from thousands of rows on through
        // registers over four waves (k_gemm_vr): alone no faster than the 16-wave kernel (1817
        // against 1810 us at 8192 rows of Dream-7B), but the whole Dream-7B lock-ramp run went
        // from 332.1-332.5 to 338.9-339.4 tokens/s with it (same box, runs alternated)
        p.bm = 256;
        p.bn = 256;
        p.wm = 4;
        p.wn = 4;
        p.pd = 12;
        p.ilv = 1;
        p.vr = M >= kVrRows;
      } else if (N % 96 == 0) {  // 96 outputs (192 interleaved gate/up rows) per tile
        p.bm = 256;
        p.bn = 192;
        p.wm = 4;
        p.wn = 3;  // 12 waves, 8 of them issuing the tile loads
        p.pd = 12;
        p.ilv = 1;
        p.vr = M >= 256;  // through registers: 1-3% faster at 512 and 820 rows
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
    const int big_splits = (K >= 2 * N) ? 2 : 1;  // long reductions (down) in two K halves
    const long row_tiles = (M + 255) / 256;
    const long big_wgs = row_tiles * (N / 256) * big_splits;
    // thousands of rows: the register-staged kernel also where its tiles give 1.5 rounds or more
    // (Dream-7B's O at 8192 rows, 448 workgroups: 212 against 226 us on 128 x 128 tiles)
    const bool vr_rows = M >= kVrRows;
    if (N % 256 == 0 && (big_wgs >= kWideTileWgs || (vr_rows && big_wgs >= 384))) {
      p.bm = 256;
      p.bn = 256;
      p.wm = 4;
      p.wn = 4;
      p.pd = 12;
      p.splits = big_splits;
      // 192 columns over 4 x 3 waves when their workgroups fill the CUs' last round better:
      // Dream-7B's QKV at 8192 rows, 768 workgroups (3 full rounds) against 576 (2.25 rounds),
      // 270.6 against 324.9 us.  Down, the only split product here, took 256 x 128 tiles over
      // 16 waves at 7 full rounds in 1148 us against 1068 on its 3.5 rounds of 256 x 256, so
      // the rule does not reach it.
      const long wgs192 = (big_splits == 1 && N % 192 == 0) ? row_tiles * (N / 192) : 0;
      if (big_wgs >= kWideTileWgs && wgs192 > 0 && round_fill(wgs192) > round_fill(big_wgs)) {
        p.bn = 192;
        p.wn = 3;
        p.vr = 1;  // through registers: Dream-7B's QKV at 8192 rows 282.5 -> 269.6 us
        return p;
      }
      // from thousands of rows on, through registers over four waves (k_gemm_vr): 4-8% faster
      // than the 16-wave kernel on every such product measured
      p.vr = vr_rows ? 1 : 0;
      return p;
    }
    if (wide) {
      p.bm = 256;
      p.bn = (N % 192 == 0) ? 192 : 256;
      p.wm = (p.bn == 192) ? 4 : 2;
      p.wn = (p.bn == 192) ? 3 : 4;
      p.pd = 12;
      // 192 columns through registers (k_gemm_vr): QKV 57.2 -> 55.0 us at 512 rows (2 K splits),
      // 105.7 -> 100.9 us at 820 rows
      p.vr = (p.bn == 192 && M >= 256) ? 1 : 0;
      target = 192;
    } else if (K >= 2 * N && N % 128 == 0 && K / (64 * 4) >= 3) {
      // long reductions into narrow outputs (the down projection): a 4-way K split, 2-way
      // once the row tiles alone give three workgroups per CU; 16 waves (64 x 32 wave tiles):
      // 117.3-117.8 against 123.9-125.1 us over 4 x 2 at 820 rows, no slower at 512
      p.bm = 256;
      p.wm = 4;
      p.wn = 4;
      p.pd = 13;
      p.splits = ((long)((M + 255) / 256) * ((N + 127) / 128) >= 768) ? 2 : 4;
      // through registers (k_gemm_vr, two 32-column blocks per wave): 60.4 -> 56.7 us at 512 rows,
      // 122.8 -> 116.6 at 820 (launches alternated, bit-identical); whole runs within their noise
      // (default generation 750.3-751.4 against 749.7-750.4 tokens/s, long-context run 471.7-473.1
      // against 473.5-474.2, same box)
      p.vr = (M >= 256) ? 1 : 0;
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

template <int BM, int BN, int NS, int EPI, int KG, int WM, int WN, int NL = 0>
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
  hipLaunchKernelGGL((k_gemm_lds<BM, BN, NS, EPI, occ, KG, WM, WN, NL>), dim3(tm * tn * p.splits), dim3(64 * KG * WM * WN), 0, s,
                     (const uint16_t*)A, (const uint16_t*)W, C, (uint16_t*)H, M, N, K, p.splits, tm, tn, n_active, k_max);
  return hipGetLastError();
}

template <int EPI, int BN>
static hipError_t launch_vr(const GemmPlan& p, const void* A, const void* W, float* C, void* H, int M, int N, int K,
                            const int32_t* n_active, int k_max, hipStream_t s) {
  // 32-bit buffer offsets within one tile: 256 rows of A, and BN weight rows (plain) or the
  // gate..up span F + BN / 2 rows (SwiGLU); every split fills the three-stage prologue; whole row
  // tiles of loads (the last one moved up), whole weight tiles
  const int ncols = EPI == 0 ? BN : BN / 2;
  const long w_span = EPI == 0 ? BN : (long)N + BN / 2;
  if (256L * K * 2 > 0x7fffffffL || w_span * K * 2 > 0x7fffffffL || K / 64 / p.splits < 3 || M < 256 || N % ncols)
    return hipErrorInvalidValue;
  const int tm = (M + 255) / 256, tn = N / ncols;
  hipLaunchKernelGGL((k_gemm_vr<EPI, BN>), dim3(tm * tn * p.splits), dim3(256), 0, s, (const uint16_t*)A,
                     (const uint16_t*)W, C, (uint16_t*)H, M, N, K, p.splits, tm, tn, n_active, k_max);
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
  if (p.vr) {
    if (p.bm != 256 || p.bk != 64 || p.ilv) return hipErrorInvalidValue;
    if (p.bn == 256) return launch_vr<0, 256>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
    if (p.bn == 192) return launch_vr<0, 192>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
    if (p.bn == 128) return launch_vr<0, 128>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
    return hipErrorInvalidValue;
  }
  // 256 x 192 over 4 x 3 wavefronts: the first 8 issue the tile loads (12 would not divide them)
  if (p.bm == 256 && p.bn == 192 && p.bk == 64 && p.pd == 12 && p.kg == 1 && p.wm == 4 && p.wn == 3)
    return launch_lds<256, 192, 2, 0, 1, 4, 3, 8>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
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
  if (p.vr) {
    if (p.bm != 256 || p.bk != 64 || !p.ilv) return hipErrorInvalidValue;
    if (p.bn == 256) return launch_vr<2, 256>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s);
    if (p.bn == 192) return launch_vr<2, 192>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s);
    return hipErrorInvalidValue;
  }
  if (p.ilv && p.bm == 256 && p.bn == 192 && p.bk == 64 && p.pd == 12 && p.kg == 1 && p.wm == 4 && p.wn == 3)
    return launch_lds<256, 192, 2, 2, 1, 4, 3, 8>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s);
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
