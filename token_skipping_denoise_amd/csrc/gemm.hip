// Active-row GEMMs: C[s][m][n] = sum_{k in split s} A[m][k] * W[n][k].
//
// ES-dLLM (technical summary 2.1 item 2) notes that computing only the
// selected rows shrinks the matrix products of the later layers: M becomes
// the number of active rows.  Both operands are K-contiguous (activations
// [M, K], nn.Linear weights [N, K]), which is the natural layout for the
// CDNA matrix cores.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation,
// 256 threads = 2x2 wavefronts, BK = 64, double-buffered LDS tiles padded to
// 72 elements per row (conflict-free 16-byte fragment reads), global loads for
// tile k+1 issued before the MFMAs of tile k.  Split-K writes fp32 partials
// that the row epilogues reduce; row tiles with no live row exit at once.
// Workgroup ids are remapped so that each XCD works on a contiguous range of
// tiles, m-tile fastest, so tiles sharing a weight panel share that XCD's L2.
//
// fp32 path (small fp32 models): LDS-tiled FMA kernel, 64x64 tiles.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;  // padded LDS row (elements)

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
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                      float* __restrict__ C, uint16_t* __restrict__ H, int M, int N,
                                                      int K, int splits, int tiles_m, int tiles_n,
                                                      const int32_t* __restrict__ n_active, int k_max) {
  constexpr int TM = BM / 64, TN = BN / 64;        // 32x32 MFMA tiles per wavefront
  constexpr int CA = BM / 32, CB = BN / 32;        // 16-byte chunks per thread per tile
  static_assert(EPI == 0 || TN % 2 == 0, "fused SwiGLU needs an even number of column blocks per wave");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLDK];

  int tmi, tni, sp;
  decode_tile(tiles_m * tiles_n * splits, tiles_m, tiles_n, tmi, tni, sp);
  const int m0 = tmi * BM;
  if (!tile_live(m0, BM, M, n_active, k_max)) return;

  const int nkb = K / kBK;
  const int kb0 = (int)((long)sp * nkb / splits), kb1 = (int)((long)(sp + 1) * nkb / splits);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // weight row feeding B-tile row c
  const int F = N;  // EPI == 1: N is the SwiGLU width F (W has 2F rows)
  const int h0 = tni * (BN / 2);
  auto w_row = [&](int c) -> int {
    if (EPI == 0) return tni * BN + c;
    const int half = c / (BN / 2), lc = c % (BN / 2);
    const int jb = lc / 32, t = lc % 32;
    return (jb < TN / 2) ? h0 + half * (BN / 4) + jb * 32 + t : F + h0 + half * (BN / 4) + (jb - TN / 2) * 32 + t;
  };
  const int w_rows = (EPI == 0) ? N : 2 * F;
  int wr[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) wr[i] = w_row((tid + 256 * i) >> 3);

  uint4 ra[2][CA], rb[2][CB];
  auto load_global = [&](int set, int kb) {
    const long k0 = (long)kb * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      const int g = m0 + row;
      ra[set][i] = (g < M) ? *reinterpret_cast<const uint4*>(A + (long)g * K + k0 + kc * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int kc = (tid + 256 * i) & 7;
      const int g = wr[i];
      rb[set][i] = (g < w_rows) ? *reinterpret_cast<const uint4*>(W + (long)g * K + k0 + kc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(&As[buf][row * kLDK + kc * 8]) = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(&Bs[buf][row * kLDK + kc * 8]) = rb[set][i];
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][(wm * (BM / 2) + i * 32 + frow) * kLDK + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][(wn * (BN / 2) + j * 32 + frow) * kLDK + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Pipeline: tiles kb+1 and kb+2 are in flight (two register sets) while tile kb is multiplied from LDS.
  const int nk = kb1 - kb0;
  if (nk > 0) {
    load_global(0, kb0);
    if (nk > 1) load_global(1, kb0 + 1);
    store_lds(0, 0);
    __syncthreads();
  }
  for (int it = 0; it < nk; it += 2) {
    // even step: compute tile it from buffer 0; set 0 is free, set 1 holds tile it+1
    if (it + 2 < nk) load_global(0, kb0 + it + 2);
    compute(0);
    if (it + 1 < nk) store_lds(1, 1);
    __syncthreads();
    if (it + 1 >= nk) break;
    // odd step: compute tile it+1 from buffer 1; set 1 is free, set 0 holds tile it+2
    if (it + 3 < nk) load_global(1, kb0 + it + 3);
    compute(1);
    if (it + 2 < nk) store_lds(0, 0);
    __syncthreads();
  }

  if (EPI == 0) {
    float* Cs = C + (long)sp * M * N;
    const int n0 = tni * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row < M) Cs[(long)row * N + col] = acc[i][j][e];
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int col = h0 + wn * (BN / 4) + j * 32 + (lane & 31);
        if (col >= F) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row >= M) continue;
          const float g = acc[i][j][e], u = acc[i][j + TN / 2][e];
          H[(long)row * F + col] = f2bf(g / (1.0f + expf(-g)) * u);
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

GemmPlan gemm_plan(int dtype, int M, int N, int K, bool swiglu) {
  GemmPlan p{64, 64, 1};
  if (dtype == 0) {
    const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
    while (!swiglu && tiles * p.splits < 256 && (K / 16) / (p.splits * 2) >= 8) p.splits *= 2;
    return p;
  }
  // Few active rows: the product streams its weights once (HBM bound); 64-row tiles
  // give two workgroups per weight panel, the second reading the panel from L2.
  p.bm = (M <= 128) ? 64 : 128;
  p.bn = (swiglu || M > 128 || N >= 16384) ? 128 : 64;
  if (swiglu) return p;  // the fused epilogue needs the whole reduction in one workgroup
  const long tiles = (long)((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  const int nkb = K / kBK;
  // split K until every CU has a workgroup, while the fp32 partial round trip
  // (8 M N bytes per split) stays under a quarter of the weight bytes when few rows are active
  for (;;) {
    const int s2 = p.splits * 2;
    if (tiles * p.splits >= 256 || nkb / s2 < 8) break;
    if (M <= 256 && 8.0 * s2 * M * (double)N > 0.25 * 2.0 * (double)N * K) break;
    if (s2 > 4) break;
    p.splits = s2;
  }
  return p;
}

template <int BM, int BN, int EPI>
static void launch_bf16(const GemmPlan& p, const void* A, const void* W, float* C, void* H, int M, int N, int K,
                        const int32_t* n_active, int k_max, hipStream_t s) {
  const int ncols = EPI == 0 ? BN : BN / 2;
  const int tm = (M + BM - 1) / BM, tn = (N + ncols - 1) / ncols;
  hipLaunchKernelGGL((k_gemm_bf16<BM, BN, EPI>), dim3(tm * tn * p.splits), dim3(256), 0, s, (const uint16_t*)A,
                     (const uint16_t*)W, C, (uint16_t*)H, M, N, K, p.splits, tm, tn, n_active, k_max);
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
  if (K % kBK != 0) return hipErrorInvalidValue;
  if (p.bm == 64 && p.bn == 64) launch_bf16<64, 64, 0>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
  else if (p.bm == 128 && p.bn == 64) launch_bf16<128, 64, 0>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
  else if (p.bm == 64 && p.bn == 128) launch_bf16<64, 128, 0>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
  else if (p.bm == 128 && p.bn == 128) launch_bf16<128, 128, 0>(p, A, W, C, nullptr, M, N, K, n_active, k_max, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu(const GemmPlan& p, const void* A, const void* W_gate_up, void* H, int M, int F, int K,
                              const int32_t* n_active, int k_max, hipStream_t s) {
  if (M <= 0 || F <= 0) return hipSuccess;
  if (K % kBK != 0 || F % (p.bn / 2) != 0 || p.splits != 1) return hipErrorInvalidValue;
  if (p.bm == 64 && p.bn == 128) launch_bf16<64, 128, 1>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s);
  else if (p.bm == 128 && p.bn == 128) launch_bf16<128, 128, 1>(p, A, W_gate_up, nullptr, H, M, F, K, n_active, k_max, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dllm
