// Bidirectional attention of the active queries over the whole K/V cache.
//
// The model family is non-causal (ES-dLLM summary section 1: every iteration
// processes the full bidirectional context).  Skipped or locked positions are
// not recomputed but stay attendable through the K/V cached when they were
// last computed (ES-dLLM 2.1 item 2; SureLock 2.1 item 3), so the cost is
// O(M_t * N * d) for M_t active rows (SureLock 2.1 item 4).
//
// bf16 kernel (gfx950 MFMA, flash style): a workgroup owns 128 queries of one
// (sequence, KV head) -- the rows x the GQA heads that share that KV head.  Its
// eight wavefronts form two groups of four; the groups take alternate 64-key
// tiles and merge their softmax states through LDS at the end.  K and V tiles
// stream from memory straight into LDS (buffer loads with an LDS destination,
// range-checked so keys past S read as zero), two stages per group, in their
// natural [key][d] layout with 16-byte chunks XOR-swizzled per row.  Scores are
// formed transposed, S^T = K Q^T, so each lane holds one query and its online-
// softmax state; the exponentiated scores then serve directly as the B operand
// of O^T += V^T P^T.  The V^T operand is read with the gfx950 transposing LDS
// read (ds_read_b64_tr_b16): in each 16-lane group, lane i receives column
// n0 + i of four consecutive rows when lane j addresses row K0 + j/4 at column
// n0 + 4 (j % 4).  The key order inside a fragment matches the accumulator
// layout of the scores (any consistent k order gives the same contraction).
// Only when few workgroups would cover a long key range is that range also
// split across workgroups (split-KV), whose partial results a second kernel
// merges.  When 128-query workgroups would leave most CUs idle (the 128 active
// rows of an early-skip layer), k_attn_q32 serves 32 query slots per workgroup
// instead, its eight waves splitting the keys (see there).  Both remap workgroup
// ids so that the query blocks of one (sequence, KV head) share an XCD's L2.
//
// fp32 kernel (small fp32 models): one wavefront per (row, head), keys one at
// a time with an online softmax.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------- fp32 ----------------
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ q, const float* __restrict__ kc,
                                                  const float* __restrict__ vc, float* __restrict__ o,
                                                  const int32_t* __restrict__ n_active, int S, int k_max, int Hq,
                                                  int Hkv, int D, float scale) {
  const int r = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int b = r / k_max, j = r - b * k_max;
  if (h >= Hq || j >= n_active[b]) return;
  const int g = Hq / Hkv, hk = h / g;
  const int nd = D / kWave;  // 1 or 2
  float qv[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  for (int t = 0; t < nd; ++t) qv[t] = q[((long)r * Hq + h) * D + lane + t * kWave];
  float m = -INFINITY, l = 0.f;
  for (int key = 0; key < S; ++key) {
    const long base = (((long)b * S + key) * Hkv + hk) * D;
    float part = 0.f;
    for (int t = 0; t < nd; ++t) part += qv[t] * kc[base + lane + t * kWave];
    const float s = wave_sum(part) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn), p = expf(s - mn);
    l = l * corr + p;
    for (int t = 0; t < nd; ++t) acc[t] = acc[t] * corr + p * vc[base + lane + t * kWave];
    m = mn;
  }
  for (int t = 0; t < nd; ++t) o[((long)r * Hq + h) * D + lane + t * kWave] = acc[t] / l;
}

// ---------------- bf16 MFMA ----------------
constexpr int kKT = 64;                       // keys per tile
constexpr int kHD = 128;                      // head dim
constexpr int kRowBytes = kHD * 2;            // one key row of K or V
constexpr int kTileBytes = kKT * kRowBytes;   // 16 KB per tensor
constexpr int kStageBytes = 2 * kTileBytes;   // K tile, then V tile
constexpr int kRing = 4;                      // stages shared by the workgroup
// Fourth word of a raw buffer resource (CDNA): 32-bit data format, no swizzle; out-of-range
// offsets read as zero.
constexpr int kBufWord3 = 0x00020000;
// Cache policy of the K/V stream: nontemporal (the long-context layer measured 93.0 against
// 95.7 us per launch with default caching).
constexpr int kNT = 2;
typedef __attribute__((address_space(3))) void lds_void;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

// 16-byte chunk c of tile row r sits in slot c ^ swz(r): the MFMA K reads (16 rows at one
// chunk) and the transposing V reads (8 rows x 4 chunks) both touch every bank once per pass.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Eight transposing 8-byte LDS reads, complete when the block ends.  Written out because the
// compiler does not know which LDS bytes the builtin reads and so waits for every direct-to-LDS
// load still in flight before it, the next tiles' included.
__device__ __forceinline__ void tr_read8(short4_t (&d)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

// The same for sixteen reads (both 16-key halves of a tile's V^T fragments).
__device__ __forceinline__ void tr_read16(short4_t (&d)[16], const uint32_t (&a)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %20\n\t"
      "ds_read_b64_tr_b16 %5, %21\n\t"
      "ds_read_b64_tr_b16 %6, %22\n\t"
      "ds_read_b64_tr_b16 %7, %23\n\t"
      "ds_read_b64_tr_b16 %8, %24\n\t"
      "ds_read_b64_tr_b16 %9, %25\n\t"
      "ds_read_b64_tr_b16 %10, %26\n\t"
      "ds_read_b64_tr_b16 %11, %27\n\t"
      "ds_read_b64_tr_b16 %12, %28\n\t"
      "ds_read_b64_tr_b16 %13, %29\n\t"
      "ds_read_b64_tr_b16 %14, %30\n\t"
      "ds_read_b64_tr_b16 %15, %31\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7]),
        "=&v"(d[8]), "=&v"(d[9]), "=&v"(d[10]), "=&v"(d[11]), "=&v"(d[12]), "=&v"(d[13]), "=&v"(d[14]),
        "=&v"(d[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]),
        "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

// Combine lanes l and l ^ 32 without an LDS round trip: v_permlane32_swap exchanges the
// upper half of one register with the lower half of another, so afterwards the two results
// hold (x[l % 32], x[l % 32 + 32]) in the same order on every lane.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  lo = __builtin_bit_cast(float, (unsigned)r[0]);
  hi = __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float half_swap_max(float x) {
  float a, b;
  half_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  float a, b;
  half_pair(x, a, b);
  return a + b;
}

// The online softmax keeps its reference maximum as an integer in the exp2 domain (the running
// max of s * scale * log2 e, rounded up).  Each weight 2^(x - m) is then a power-of-two multiple
// of its value against any other integer reference, so its bf16 rounding (the matrix-core
// operand of the V product) and every rescale or merge factor 2^(m_a - m_b) are exact scalings:
// the output does not depend on how the keys are split over waves, key groups or workgroups.
__device__ __forceinline__ float pow2_int(float e) { return __builtin_amdgcn_ldexpf(1.f, (int)e); }

// Reference update of one tile: when some query of the wave would see a weight above 2^8, every
// lane moves its reference to max(m, ceil(tile max)) and rescales its sum and accumulators by
// the exact power of two; otherwise nothing changes.  mt2: this lane's tile max in the exp2
// domain (-inf without a finite score).
template <int NACC>
__device__ __forceinline__ void softmax_reference(float mt2, float& m_ref, float& l_run, f32x16_t (&oacc)[NACC]) {
  if (__builtin_amdgcn_ballot_w64(mt2 > m_ref + 8.f) != 0) {
    const float m_new = fmaxf(m_ref, ceilf(mt2));
    // an empty state (m = -inf: no finite score yet) has nothing to rescale
    const float corr = (m_ref == -INFINITY || m_new == -INFINITY) ? 0.f : pow2_int(m_ref - m_new);
    l_run *= corr;
    m_ref = m_new;
#pragma unroll
    for (int db = 0; db < NACC; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
  }
}

// Workgroup coordinates with the query blocks of one (sequence, KV head) kept on one XCD.
// Workgroups are dealt to the eight XCDs in turn by linear id; when the grid is a multiple of 8,
// XCD x takes the x-th contiguous eighth of the (query block fastest) work list instead, so the
// query blocks that stream the same K/V share that XCD's L2 rather than each fetching it.
__device__ __forceinline__ void attn_block(int& bx, int& by, int& bz) {
  const int nx = gridDim.x, ny = gridDim.y;
  const int n = nx * ny * gridDim.z;
  int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  if ((n & 7) == 0) lin = (lin & 7) * (n >> 3) + (lin >> 3);
  bx = lin % nx;
  by = (lin / nx) % ny;
  bz = lin / (nx * ny);
}

template <int N>
__device__ __forceinline__ void wait_vm_attn() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// With nsplit > 1 the key tiles are divided among nsplit workgroups (split-KV): each writes
// its unnormalised output and softmax statistics (max, sum, in the exp2 domain) to `part`,
// and k_attn_merge combines them.
__global__ __launch_bounds__(512, 1) void k_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                      const uint16_t* __restrict__ vc, uint16_t* __restrict__ o,
                                                      const int32_t* __restrict__ n_active, int S, int k_max, int Hq,
                                                      int Hkv, float scale_log2e, int nsplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing * kStageBytes];  // 128 KB
  int bx, by, bz;
  attn_block(bx, by, bz);
  const int b = bz / nsplit, split = bz - b * nsplit, hk = by;
  const int g = Hq / Hkv;
  const int qb0 = bx * 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;

  // this workgroup's key tiles [t_begin, t_end); key group grp takes keys 32 grp .. 32 grp + 31
  // of every tile
  const int ntiles_all = (S + kKT - 1) / kKT;
  const int t_begin = (int)((long)split * ntiles_all / nsplit), t_end = (int)((long)(split + 1) * ntiles_all / nsplit);
  const int n_tiles = t_end - t_begin;

  // the queries first, straight into the ring's last stage (the prologue below fills the
  // others; the tile loop first writes it after its first barrier): 128 query rows of 256 B, four
  // 4-row load instructions per wave, chunk c of row r in slot c ^ swz(r) as for the tiles
  const int kq = k_max * g;
  uint8_t* qst = smem + (kRing - 1) * kStageBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (wave * 4 + i) + (lane >> 4);
    const int qs = min(qb0 + r, kq - 1);
    const int jr = qs / g;
    const long qrow_r = ((long)b * k_max + jr) * Hq + hk * g + (qs - jr * g);
    const uint16_t* src = q + qrow_r * kHD + (((lane & 15) ^ swz(r)) << 3);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(qst + (wave * 4 + i) * 1024), 16, 0, 0);
  }
  const int qi = qb0 + gw * 32 + l32;  // this lane's query slot

  // K/V tile loads: 16 load instructions of 4 rows (1 KB) per tensor, 2 per wave.  Lane L of
  // instruction qi fills row 4 qi + L / 16, slot L % 16, so it fetches chunk slot ^ swz(row).
  const long head0 = ((long)b * S * Hkv + hk) * kHD;
  const int nbytes = S * Hkv * kRowBytes;
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + head0), (short)0, nbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + head0), (short)0, nbytes, kBufWord3);
  int voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 4 * (wave * 2 + i) + (lane >> 4);
    voff[i] = row * Hkv * kRowBytes + (((lane & 15) ^ swz(row)) << 4);
  }
  const int tile_bytes = kKT * Hkv * kRowBytes;
  auto issue = [&](int t, int slot) {
    uint8_t* st = smem + slot * kStageBytes;
    const int so = t * tile_bytes;  // in the per-lane offset, which the range check covers
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qi2 = wave * 2 + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsk, (lds_void*)(st + qi2 * 1024), 16, voff[i] + so, 0, 0, kNT);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsv, (lds_void*)(st + kTileBytes + qi2 * 1024), 16, voff[i] + so, 0, 0,
                                               kNT);
    }
  };
  // the first tiles are requested before the active-row count is known (all addresses are valid
  // either way), so those round trips overlap
#pragma unroll
  for (int j = 0; j < kRing - 1; ++j)
    if (j < n_tiles) issue(t_begin + j, j);
  const int nq = n_active[b] * g;
  if (qb0 >= nq) {
    wait_vm_attn<0>();  // no load may still be writing this workgroup's LDS when it ends
    return;
  }
  // the query rows have landed once at most the prologue's tile loads are outstanding (loads
  // complete in order); after the barrier every wave takes its B fragments from LDS
  {
    const int np = min(kRing - 1, n_tiles);
    if (np >= 3) wait_vm_attn<12>();
    else if (np == 2) wait_vm_attn<8>();
    else if (np == 1) wait_vm_attn<4>();
    else wait_vm_attn<0>();
  }
  __builtin_amdgcn_s_barrier();
  bf16x8_t qf[kHD / 16];
  {
    const int r = gw * 32 + l32;
    const uint8_t* rp = qst + r * kRowBytes;
#pragma unroll
    for (int t = 0; t < kHD / 16; ++t) qf[t] = *reinterpret_cast<const bf16x8_t*>(rp + (((2 * t + hi) ^ swz(r)) << 4));
  }
  // the reads are done before the first tile loop barrier lets a load overwrite the stage
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  // a query slot past the live rows computes on whatever its row holds; its lanes never mix
  // with other queries' lanes and are not written back
  const bool qvalid = qi < nq;

  f32x16_t oacc[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  // integer reference in the exp2 domain, and the softmax sum of 2^(s * scale_log2e - m)
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane parts of the fragment addresses
  const int k_row = grp * 32 + l32;
  const int k_sw = swz(k_row);
  const int v_row = grp * 32 + 4 * hi + ((lane & 15) >> 2);    // + 16 hf (+ 8)
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 db
  // byte offsets (within a stage's V tile) of the sixteen transposing reads: half hf of the
  // tile's 32 keys, column block db, rows r0 (keys +0..3) and r0 + 8 (keys +8..11)
  uint32_t v_off[16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r0 = 16 * hf + v_row, r1 = r0 + 8;
    const int sw0 = swz(r0), sw1 = swz(r1);
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db) {
      const int col = 32 * db + v_col;  // element column of this lane's 8-byte read
      const int inb = (col & 7) << 1;   // byte within the 16-byte chunk
      v_off[8 * hf + 2 * db] = r0 * kRowBytes + ((((col >> 3) ^ sw0) << 4) | inb);
      v_off[8 * hf + 2 * db + 1] = r1 * kRowBytes + ((((col >> 3) ^ sw1) << 4) | inb);
    }
  }
  for (int i = 0; i < n_tiles; ++i) {
    // tiles after i may stay in flight (2 loads per tensor per wave each)
    const int ahead = min(kRing - 2, n_tiles - 1 - i);
    if (ahead >= 2) wait_vm_attn<8>();
    else if (ahead == 1) wait_vm_attn<4>();
    else wait_vm_attn<0>();
    __builtin_amdgcn_s_barrier();  // every wave's loads of tile i have landed; slot (i - 1) is free
    if (i + kRing - 1 < n_tiles) issue(t_begin + i + kRing - 1, (i + kRing - 1) % kRing);
    const int t = t_begin + i;
    const uint8_t* kst = smem + (i % kRing) * kStageBytes;
    const uint8_t* vst = kst + kTileBytes;
    // S^T for this group's 32 keys of the tile
    f32x16_t sacc;
    short4_t tv[16];
    {
      const uint8_t* rp = kst + k_row * kRowBytes;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
      // every LDS read of the tile in one batch, so the wave waits for LDS once per tile: the
      // eight K fragments, then the sixteen transposing V^T reads, whose block ends with the wait
      bf16x8_t kf[kHD / 16];
#pragma unroll
      for (int ts = 0; ts < kHD / 16; ++ts) kf[ts] = *reinterpret_cast<const bf16x8_t*>(rp + (((2 * ts + hi) ^ k_sw) << 4));
      const uint32_t vb = lds_addr(vst);
      uint32_t ad[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ad[j] = vb + v_off[j];
      tr_read16(tv, ad);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads together (the scheduler would spread them)
#pragma unroll
      for (int ts = 0; ts < kHD / 16; ++ts) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ts], qf[ts], sacc, 0, 0, 0);
    }
    // the last tile may be partial: keys past S score -inf
    const int key0 = t * kKT + grp * 32;
    if (key0 + 32 > S) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 8 * (e >> 2) + 4 * hi + (e & 3) >= S) sacc[e] = -INFINITY;
    }
    // online softmax (each query lives in lanes l and l^32)
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[e]);
    mt = half_swap_max(mt);
    // The reference only moves when some query of the wave would otherwise see a weight above
    // 2^8; below that, numerator and sum keep the old reference, which saves rescaling the
    // accumulators on almost every tile (the weights are exact power-of-two multiples either way).
    softmax_reference(mt * scale_log2e, m_run, l_run, oacc);
    // m_run = -inf only while every score seen is -inf, so every weight is 0 then
    const float mc = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2e, -mc));
      sacc[e] = p;
      rs += p;
    }
    rs = half_swap_sum(rs);
    l_run += rs;

    // O^T += V^T P^T over two 16-key steps; the V^T fragment of half hf and column block db
    // (keys r0..r0+3 and r0+8..r0+11 of column 32 db + l32) is the pair of transposing reads
    // 8 hf + 2 db and 8 hf + 2 db + 1 made above
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2_t pr = {sacc[8 * hf + 2 * e], sacc[8 * hf + 2 * e + 1]};
        pw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
      }
      const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db) {
        const short4_t lo = tv[8 * hf + 2 * db], hv = tv[8 * hf + 2 * db + 1];
        const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hv[0], hv[1], hv[2], hv[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8), pfrag, oacc[db], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before it is reused below

  // merge group 1 into group 0 through LDS: float4 [wave][db][e4][lane] (64 KB), then (m, l)
  // per wave lane
  float4* xs = reinterpret_cast<float4*>(smem);
  float* ml = reinterpret_cast<float*>(smem + 4 * (kHD / 32) * 4 * 64 * sizeof(float4));
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        xs[((gw * (kHD / 32) + db) * 4 + e4) * 64 + lane] =
            make_float4(oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]);
    ml[(gw * 2) * 64 + lane] = m_run;
    ml[(gw * 2 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = ml[(gw * 2) * 64 + lane], l1 = ml[(gw * 2 + 1) * 64 + lane];
    const float M = fmaxf(m_run, m1);
    // both -inf only for a group without keys; keep the merged state finite then
    const float c0 = (m_run == -INFINITY) ? 0.f : pow2_int(m_run - M);
    const float c1 = (m1 == -INFINITY) ? 0.f : pow2_int(m1 - M);
    l_run = l_run * c0 + l1 * c1;
    m_run = M;
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float4 x = xs[((gw * (kHD / 32) + db) * 4 + e4) * 64 + lane];
        oacc[db][4 * e4] = oacc[db][4 * e4] * c0 + x.x * c1;
        oacc[db][4 * e4 + 1] = oacc[db][4 * e4 + 1] * c0 + x.y * c1;
        oacc[db][4 * e4 + 2] = oacc[db][4 * e4 + 2] * c0 + x.z * c1;
        oacc[db][4 * e4 + 3] = oacc[db][4 * e4 + 3] * c0 + x.w * c1;
      }
  }

  if (nsplit > 1) {
    if (!qvalid) return;
    const int jrow = qi / g;
    const long qrow = (long)b * k_max + jrow;
    const int h = hk * g + (qi - jrow * g);
    // partial layout: [split][row][head][D + 2] = unnormalised O, then (m, l)
    const long n_rows = (long)(gridDim.z / nsplit) * k_max;  // B * k_max
    float* pp = part + (((long)split * n_rows + qrow) * Hq + h) * (kHD + 2);
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * hi;
        *reinterpret_cast<float2*>(pp + d) = make_float2(oacc[db][4 * e4], oacc[db][4 * e4 + 1]);
        *reinterpret_cast<float2*>(pp + d + 2) = make_float2(oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]);
      }
    if (hi == 0) {
      pp[kHD] = m_run;  // the integer reference, exp2 domain
      pp[kHD + 1] = l_run;
    }
    return;
  }
  if (!qvalid) return;
  const int jrow = qi / g;
  const long qrow = (long)b * k_max + jrow;
  const int h = hk * g + (qi - jrow * g);
  const float inv_l = 1.0f / l_run;
  uint16_t* op = o + (qrow * Hq + h) * kHD;
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = db * 32 + 8 * e4 + 4 * hi;
      const uint32_t w0 = pack_bf16x2(oacc[db][4 * e4] * inv_l, oacc[db][4 * e4 + 1] * inv_l);
      const uint32_t w1 = pack_bf16x2(oacc[db][4 * e4 + 2] * inv_l, oacc[db][4 * e4 + 3] * inv_l);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

// ---- short key ranges: 32 query slots per workgroup, keys split among its waves ----
// With a few hundred keys, a workgroup of 128 queries spends most of its time in the latency
// of one tile after the next while most CUs have nothing to do.  Here a workgroup owns 32
// query slots of one (sequence, KV head) -- four times the workgroups -- and each of its
// kQWaves wavefronts takes a contiguous share of the 32-key tiles through an LDS ring of its own
// (kQRing stages), so no wave waits for another until the softmax states are merged at the end
// (each wave then finishes 16 / kQWaves of the output's 32 x 8-column groups).  The per-tile
// arithmetic is that of k_attn_bf16.  Eight waves with one stage each keep as many tiles in
// flight per CU as four waves with two but from twice the issuing waves: 8.8-9.3 against
// 9.8-9.9 us per launch on the LLaDA-8B layer over 128 rows at S = 512.
constexpr int kQT = 32;                       // keys per tile
constexpr int kQTileBytes = kQT * kRowBytes;  // 8 KB per tensor
constexpr int kQStage = 2 * kQTileBytes;      // K tile, then V tile
constexpr int kQWavesUsed = 8, kQRingUsed = 1;

template <int kQWaves, int kQRing>
__global__ __launch_bounds__(64 * kQWaves, 1) void k_attn_q32(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                     const uint16_t* __restrict__ vc, uint16_t* __restrict__ o,
                                                     const int32_t* __restrict__ n_active, int S, int k_max, int Hq,
                                                     int Hkv, float scale_log2e) {
  // four per-wave rings (128 KB), then the 32 query rows (8 KB)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kQWaves * kQRing * kQStage + kQT * kRowBytes];
  static_assert(8 % kQWaves == 0 && 16 % kQWaves == 0, "query loads and output pairs split evenly over the waves");
  static_assert(kQWaves * ((kHD / 32) * 4 * 64 * 16 + 2 * 64 * 4) <= (int)sizeof(smem), "the merge fits the LDS");
  int bx, by, bz;
  attn_block(bx, by, bz);
  const int b = bz, hk = by;
  const int g = Hq / Hkv;
  const int qb0 = bx * 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int ntiles_all = (S + kQT - 1) / kQT;
  const int t_begin = wave * ntiles_all / kQWaves, t_end = (wave + 1) * ntiles_all / kQWaves;
  const int n_tiles = t_end - t_begin;
  uint8_t* ring = smem + wave * kQRing * kQStage;
  uint8_t* qst = smem + kQWaves * kQRing * kQStage;

  // the 32 query rows: eight 4-row load instructions, 8 / kQWaves per wave, chunk c of row r in
  // slot c ^ swz(r)
  const int kq = k_max * g;
  constexpr int QPW = 8 / kQWaves;
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int r = 4 * (wave * QPW + i) + (lane >> 4);
    const int qs = min(qb0 + r, kq - 1);
    const int jr = qs / g;
    const long qrow_r = ((long)b * k_max + jr) * Hq + hk * g + (qs - jr * g);
    const uint16_t* src = q + qrow_r * kHD + (((lane & 15) ^ swz(r)) << 3);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(qst + (wave * QPW + i) * 1024), 16, 0, 0);
  }

  // K/V tiles: eight 4-row load instructions per tensor, all issued by the owning wave; lane L
  // of instruction i fills row 4 i + L / 16, slot L % 16, so it fetches chunk slot ^ swz(row)
  const long head0 = ((long)b * S * Hkv + hk) * kHD;
  const int nbytes = S * Hkv * kRowBytes;
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + head0), (short)0, nbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + head0), (short)0, nbytes, kBufWord3);
  int voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4);
    voff[i] = row * Hkv * kRowBytes + (((lane & 15) ^ swz(row)) << 4);
  }
  const int tile_bytes = kQT * Hkv * kRowBytes;
  auto issue = [&](int t, int slot) {
    uint8_t* st = ring + slot * kQStage;
    const int so = t * tile_bytes;  // in the per-lane offset, which the range check covers
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsk, (lds_void*)(st + i * 1024), 16, voff[i] + so, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsv, (lds_void*)(st + kQTileBytes + i * 1024), 16, voff[i] + so, 0, 0,
                                               0);
    }
  };
#pragma unroll
  for (int j = 0; j < kQRing; ++j)
    if (j < n_tiles) issue(t_begin + j, j);
  const int nq = n_active[b] * g;
  if (qb0 >= nq) {
    wait_vm_attn<0>();  // no load may still be writing this workgroup's LDS when it ends
    return;
  }
  // the query rows have landed once at most the tile loads (16 per tile) are outstanding
  {
    const int np = min(kQRing, n_tiles);
    if (np >= 2) wait_vm_attn<32>();
    else if (np == 1) wait_vm_attn<16>();
    else wait_vm_attn<0>();
  }
  __builtin_amdgcn_s_barrier();
  bf16x8_t qf[kHD / 16];
  {
    const uint8_t* rp = qst + l32 * kRowBytes;
#pragma unroll
    for (int t = 0; t < kHD / 16; ++t) qf[t] = *reinterpret_cast<const bf16x8_t*>(rp + (((2 * t + hi) ^ swz(l32)) << 4));
  }
  const int qi = qb0 + l32;  // this lane's query slot
  const bool qvalid = qi < nq;

  f32x16_t oacc[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // integer exp2-domain reference, softmax sum

  const int k_sw = swz(l32);
  const int v_row = 4 * hi + ((lane & 15) >> 2);              // + 16 hf (+ 8)
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32 db
  uint32_t v_off[16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r0 = 16 * hf + v_row, r1 = r0 + 8;
    const int sw0 = swz(r0), sw1 = swz(r1);
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db) {
      const int col = 32 * db + v_col;
      const int inb = (col & 7) << 1;
      v_off[8 * hf + 2 * db] = r0 * kRowBytes + ((((col >> 3) ^ sw0) << 4) | inb);
      v_off[8 * hf + 2 * db + 1] = r1 * kRowBytes + ((((col >> 3) ^ sw1) << 4) | inb);
    }
  }
  for (int i = 0; i < n_tiles; ++i) {
    if (kQRing >= 2 && i + 1 < n_tiles) wait_vm_attn<16>();  // tile i + 1 may stay in flight
    else wait_vm_attn<0>();
    const int t = t_begin + i;
    const uint8_t* kst = ring + (i % kQRing) * kQStage;
    f32x16_t sacc;
    short4_t tv[16];
    bf16x8_t kf[kHD / 16];
    {
      const uint8_t* rp = kst + l32 * kRowBytes;
#pragma unroll
      for (int ts = 0; ts < kHD / 16; ++ts) kf[ts] = *reinterpret_cast<const bf16x8_t*>(rp + (((2 * ts + hi) ^ k_sw) << 4));
      const uint32_t vb = lds_addr(kst + kQTileBytes);
      uint32_t ad[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ad[j] = vb + v_off[j];
      tr_read16(tv, ad);  // ends with the LDS wait, so the stage is free afterwards
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i + kQRing < n_tiles) issue(t + kQRing, i % kQRing);
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
    for (int ts = 0; ts < kHD / 16; ++ts) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ts], qf[ts], sacc, 0, 0, 0);
    const int key0 = t * kQT;
    if (key0 + kQT > S) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key0 + 8 * (e >> 2) + 4 * hi + (e & 3) >= S) sacc[e] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[e]);
    mt = half_swap_max(mt);
    softmax_reference(mt * scale_log2e, m_run, l_run, oacc);
    const float mc = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2e, -mc));
      sacc[e] = p;
      rs += p;
    }
    rs = half_swap_sum(rs);
    l_run += rs;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(sacc[8 * hf + 2 * e], sacc[8 * hf + 2 * e + 1]);
      const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db) {
        const short4_t lo = tv[8 * hf + 2 * db], hv = tv[8 * hf + 2 * db + 1];
        const short8_t a8 = {lo[0], lo[1], lo[2], lo[3], hv[0], hv[1], hv[2], hv[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8), pfrag, oacc[db], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with its ring before the rings are reused below

  // merge: every wave leaves its O^T fragments (float4 [wave][db][e4][lane], 64 KB) and (m, l);
  // wave w then combines the four states for column block w
  float4* xs = reinterpret_cast<float4*>(smem);
  float* ml = reinterpret_cast<float*>(smem + kQWaves * (kHD / 32) * 4 * 64 * sizeof(float4));
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      xs[((wave * (kHD / 32) + db) * 4 + e4) * 64 + lane] =
          make_float4(oacc[db][4 * e4], oacc[db][4 * e4 + 1], oacc[db][4 * e4 + 2], oacc[db][4 * e4 + 3]);
  ml[(wave * 2) * 64 + lane] = m_run;
  ml[(wave * 2 + 1) * 64 + lane] = l_run;
  __syncthreads();
  float mw[kQWaves], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kQWaves; ++w) {
    mw[w] = ml[(w * 2) * 64 + lane];
    M = fmaxf(M, mw[w]);
  }
  float cw[kQWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kQWaves; ++w) {
    // a wave without keys (or with only masked ones) keeps m = -inf and contributes nothing
    cw[w] = (mw[w] == -INFINITY) ? 0.f : pow2_int(mw[w] - M);
    L += ml[(w * 2 + 1) * 64 + lane] * cw[w];
  }
  if (!qvalid) return;
  const int jrow = qi / g;
  const long qrow = (long)b * k_max + jrow;
  const int h = hk * g + (qi - jrow * g);
  const float inv_l = 1.0f / L;
  uint16_t* op = o + (qrow * Hq + h) * kHD;
  // the 16 (column block, 8-column group) pairs of the output, 16 / kQWaves per wave
  constexpr int PPW = 16 / kQWaves;
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int pr = wave * PPW + k, db = pr >> 2, e4 = pr & 3;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kQWaves; ++w) {
      const float4 x = xs[((w * (kHD / 32) + db) * 4 + e4) * 64 + lane];
      acc.x += x.x * cw[w];
      acc.y += x.y * cw[w];
      acc.z += x.z * cw[w];
      acc.w += x.w * cw[w];
    }
    const int d = db * 32 + 8 * e4 + 4 * hi;
    *reinterpret_cast<uint2*>(op + d) =
        make_uint2(pack_bf16x2(acc.x * inv_l, acc.y * inv_l), pack_bf16x2(acc.z * inv_l, acc.w * inv_l));
  }
}

// Combine split-KV partials: O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) (exact powers of two).
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, int nsplit, long split_stride,
                                                    const int32_t* __restrict__ n_active, int k_max, int Hq,
                                                    uint16_t* __restrict__ o) {
  const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int b = r / k_max, j = r - b * k_max;
  if (j >= n_active[b]) return;
  const float* p0 = part + ((long)r * Hq + h) * (kHD + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, p0[sp * split_stride + kHD]);
  float L = 0.f, acc = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* ps = p0 + sp * split_stride;
    const float w = (ps[kHD] == -INFINITY) ? 0.f : pow2_int(ps[kHD] - M);  // integer references
    L += ps[kHD + 1] * w;
    acc += ps[d] * w;
  }
  o[((long)r * Hq + h) * kHD + d] = f2bf(acc / L);
}

// The 32-query kernel when 128-query workgroups would occupy at most a quarter of the CUs
// (measured on the LLaDA-8B shapes: 128 active rows of 32 heads, S 256 .. 2048).
static bool attention_q32(int B, int k_max, int Hq, int Hkv) {
  const long wgs128 = (long)((k_max * (Hq / Hkv) + 127) / 128) * Hkv * B;
  return wgs128 <= 64;
}

// Split-KV only pays when few workgroups would each stream a long key range: a split's
// partial (128 queries x (D + 2) fp32) must stay small beside the K/V it summarises.
int attention_splits(int dtype, int B, int S, int k_max, int Hq, int Hkv) {
  if (dtype == 0 || attention_q32(B, k_max, Hq, Hkv)) return 1;
  const int g = Hq / Hkv;
  const long wgs = (long)((k_max * g + 127) / 128) * Hkv * B;
  int ns = 1;
  while (ns < 8 && wgs * ns < 128 && S / (ns * 2) >= 512) ns *= 2;
  return ns;
}

size_t attention_part_bytes(int dtype, int B, int S, int k_max, int Hq, int Hkv) {
  const int ns = attention_splits(dtype, B, S, k_max, Hq, Hkv);
  return ns > 1 ? (size_t)ns * B * k_max * Hq * (kHD + 2) * sizeof(float) : 0;
}

hipError_t launch_attention(int dtype, const void* q, const void* kc, const void* vc, void* o,
                            const int32_t* n_active, int B, int S, int k_max, int Hq, int Hkv, int D, float* part,
                            hipStream_t s) {
  if (B <= 0 || k_max <= 0) return hipSuccess;
  if (dtype == 0) {
    if (D % kWave != 0 || D > 2 * kWave) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_f32, dim3(B * k_max, (Hq + 3) / 4), dim3(256), 0, s, (const float*)q, (const float*)kc,
                       (const float*)vc, (float*)o, n_active, S, k_max, Hq, Hkv, D, 1.0f / sqrtf((float)D));
    return hipGetLastError();
  }
  if (D != kHD) return hipErrorInvalidValue;
  if ((long)S * Hkv * kHD * 2 >= (1L << 31)) return hipErrorInvalidValue;  // 32-bit buffer offsets
  const int g = Hq / Hkv;
  const int qblocks = (k_max * g + 127) / 128;
  const float scale_log2e = (float)(1.0 / sqrt((double)D) * 1.4426950408889634);
  if (attention_q32(B, k_max, Hq, Hkv)) {
    hipLaunchKernelGGL((k_attn_q32<kQWavesUsed, kQRingUsed>), dim3((k_max * g + 31) / 32, Hkv, B),
                       dim3(64 * kQWavesUsed), 0, s, (const uint16_t*)q,
                       (const uint16_t*)kc, (const uint16_t*)vc, (uint16_t*)o, n_active, S, k_max, Hq, Hkv, scale_log2e);
    return hipGetLastError();
  }
  const int ns = attention_splits(dtype, B, S, k_max, Hq, Hkv);
  if (ns > 1 && !part) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_bf16, dim3(qblocks, Hkv, B * ns), dim3(512), 0, s, (const uint16_t*)q, (const uint16_t*)kc,
                     (const uint16_t*)vc, (uint16_t*)o, n_active, S, k_max, Hq, Hkv, scale_log2e, ns, part);
  if (ns > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(B * k_max, Hq), dim3(kHD), 0, s, part, ns, (long)B * k_max * Hq * (kHD + 2),
                       n_active, k_max, Hq, (uint16_t*)o);
  return hipGetLastError();
}

}  // namespace dllm
