// Launch wrappers of the libdllm kernels (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

// ---------------- row kernels (rowops.hip) ----------------
// x[r] = embed[tok[r]] for r < rows; if g: xn[r] = rmsnorm(x[r]) * g.
// chk (debug build): error word for out-of-range token ids, or null.
hipError_t launch_embed_norm(int dtype, const void* embed, const int32_t* tokens, int V, int rows, int d,
                             const void* g, float eps, void* x, void* xn, hipStream_t s, uint32_t* chk = nullptr);
// dst[r] = src[row_pos[r]] for live rows; if g: dst_norm[r] = rmsnorm(dst[r]) * g; if dst_at_src:
// dst_at_src[row_pos[r]] = src[row_pos[r]] as well (the same rows copied in place to another buffer).
hipError_t launch_gather_norm(int dtype, const void* src, const int32_t* row_pos, int R, int w, void* dst,
                              const void* g, float eps, void* dst_norm, hipStream_t s, void* dst_at_src = nullptr);
// dst[row_pos[r]] = src[r] for live rows; if g: dst_norm[r] = rmsnorm(src[r]) * g.
hipError_t launch_scatter_norm(int dtype, const void* src, const int32_t* row_pos, int R, int w, void* dst,
                               const void* g, float eps, void* dst_norm, hipStream_t s);
// row_pos[b*k_max + j] = b*S + idx[b*k_max + j] if j < n_active[b], else -1.
// chk (debug build): error word for an active count outside [0, k_max], live indices outside
// [0, S) or not strictly ascending, or null.
hipError_t launch_row_pos(const int32_t* idx, const int32_t* n_active, int B, int S, int k_max,
                          int32_t* row_pos, hipStream_t s, uint32_t* chk = nullptr);
// idx[b*S + i] = i, n_active[b] = S; if row_pos: row_pos[b*S + i] = b*S + i.
hipError_t launch_identity_rows(int B, int S, int32_t* idx, int32_t* n_active, hipStream_t s,
                                int32_t* row_pos = nullptr);
// Sum split-K partials of the QKV GEMM, apply RoPE at position row_pos % S, write Q [R, Hq*D]
// and K/V rows into the caches [B, S, Hkv, D].
hipError_t launch_qkv_epilogue(int dtype, const float* part, int splits, long split_stride,
                               const int32_t* row_pos, int R, int S, int Hq, int Hkv, int D, float rope_base,
                               void* q, void* kc, void* vc, hipStream_t s);
// x[r] += sum of partials; if g: xn[r] = rmsnorm(x[r]) * g; if x_scatter: x_scatter[row_pos[r]] = x[r]
// as well (the new rows also written to their positions in a full-height buffer).
hipError_t launch_resid_norm(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                             int R, int d, void* x, const void* g, float eps, void* xn, hipStream_t s,
                             void* x_scatter = nullptr);
// h[r, c] = silu(P[r, c]) * P[r, F + c] with P the summed partials [R, 2F].
hipError_t launch_swiglu(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                         int R, int F, void* h, hipStream_t s);
// dst[r] = sum of the split-K partials of row r, stored in the element type (rows with row_pos >= 0).
hipError_t launch_sum_store(int dtype, const float* part, int splits, long split_stride, const int32_t* row_pos,
                            int R, int w, void* dst, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

// ---------------- GEMM (gemm.hip) ----------------
// C[s][m][n] = sum_{k in split s} A[m][k] * W[n][k] (fp32 partials, split stride M*N).
// Row tiles whose rows are all dead (j >= n_active[b], r = b*k_max + j) are skipped;
// n_active == nullptr means every row is live.
struct GemmPlan {
  int bm, bn, splits, bk, pd;  // tile rows, tile columns, K splits, K tile, 10 + LDS stages (bf16)
  int kg = 1;                  // k-groups of wavefronts per workgroup (bf16)
  int wm = 2, wn = 2;          // wavefronts along the tile's rows and columns (bf16)
  int ilv = 0;                 // SwiGLU: gate/up rows interleaved in 16s inside each 32-row block
  int vr = 0;                  // 256 x 256 tiles through registers over four waves (k_gemm_vr)
};
GemmPlan gemm_plan(int dtype, int M, int N, int K, bool swiglu = false);
hipError_t launch_gemm(int dtype, const GemmPlan& p, const void* A, const void* W, float* C, int M, int N, int K,
                       const int32_t* n_active, int k_max, hipStream_t s);
// H[m][f] = silu(sum_k A[m][k] Wg[f][k]) * sum_k A[m][k] Wu[f][k], W_gate_up = [Wg; Wu] (bf16 only).
hipError_t launch_gemm_swiglu(const GemmPlan& p, const void* A, const void* W_gate_up, void* H, int M, int F, int K,
                              const int32_t* n_active, int k_max, hipStream_t s);

// ---------------- products on fragment-packed weights (gemm_packed.hip) ----------------
// W [N, K] repacked into 1 KB MFMA B fragments (32 columns x 16 reduction elements); with
// F > 0 (the stacked [gate; up] [2F, K]) gate and up rows interleave in 16s.
hipError_t launch_pack_frag(const void* W, void* Wp, int N, int K, int F, hipStream_t s);
struct PackedPlan {
  bool ok = false;
  int nw = 0;      // waves per workgroup, one 32-column block each
  int splits = 1;  // K splits (fp32 partials)
  int nkc = 0;     // 64-element stages of the longest split
};
// Whether (and how) the packed path covers an M x N x K product (M <= 128).
PackedPlan packed_plan(int M, int N, int K, bool swiglu);
// The same for a product whose consumer needs whole sums in C (no K split): the LM head.
PackedPlan packed_plan_whole(int M, int N, int K);
// swiglu (H non-null): H[m][f] = silu(A Wg^T) * (A Wu^T), N = 2F packed columns; else fp32 partials
// C[sp][m][n].
hipError_t launch_gemm_packed(const PackedPlan& p, const void* A, const void* Wp, float* C, void* H, int M, int N,
                              int K, int F, const int32_t* n_active, int k_max, hipStream_t s);

// ---------------- attention (attention.hip) ----------------
// o[r, h, :] = softmax(q[r, h] . Kc[b, :, h/g] / sqrt(D)) Vc[b, :, h/g] over all S keys.
// Split-KV (bf16, few query blocks): `part` needs attention_part_bytes(...) bytes.
int attention_splits(int dtype, int B, int S, int k_max, int Hq, int Hkv);
size_t attention_part_bytes(int dtype, int B, int S, int k_max, int Hq, int Hkv);
hipError_t launch_attention(int dtype, const void* q, const void* kc, const void* vc, void* o,
                            const int32_t* n_active, int B, int S, int k_max, int Hq, int Hkv, int D, float* part,
                            hipStream_t s);

// ---------------- score / select (score_select.hip) ----------------
hipError_t launch_score(int dtype, const void* h_cur, const void* h_prev, void* h_next, const float* conf_prev,
                        const float* kl_prev, const uint8_t* force, int rows, int width, float alpha,
                        int conf_inverted, int var, float* score, hipStream_t s);
// Nested boundary: score of the active rows (x_act row r at position row_pos[r]) against the
// per-layer cache h_cache [positions, width]; force_nested [positions] is set to excluded except
// at the active positions, row_of [positions] maps an active position to its row (score_select.hip).
hipError_t launch_score_rows(int dtype, const void* x_act, const int32_t* row_pos, int R, const void* h_cache,
                             const float* conf_prev, const float* kl_prev, const uint8_t* force, long positions,
                             int width, float alpha, int conf_inverted, int var, float* score, uint8_t* force_nested,
                             int32_t* row_of, hipStream_t s);
// old_row[r] = row_of[row_pos[r]] (or -1 for a dead row).
hipError_t launch_compose_rows(const int32_t* row_pos, const int32_t* row_of, int R, int32_t* old_row, hipStream_t s);
hipError_t launch_select(const float* score, const uint8_t* force, int B, int S, int sel, int k, float tau,
                         int k_max, int32_t* idx, int32_t* n_active, hipStream_t s, int32_t* row_pos = nullptr);

// ---------------- vocabulary pass (vocab.hip) ----------------
// Rows are split into vocabulary slices when few rows are active; `partial` needs
// conf_kl_part_bytes(R, V) bytes (may be null when that is 0).
size_t conf_kl_part_bytes(int R, int V);
// logits_prev holds fp32 (prev_dtype 0) or bf16 (prev_dtype 1) previous logits, or is null.
hipError_t launch_conf_kl(const float* logits, void* logits_prev, int prev_dtype, const int32_t* row_pos, int R,
                          int V, int exclude_id, int have_prev, float* conf, int32_t* argmax, float* kl, void* partial,
                          hipStream_t s);

// ---------------- achievable-peak probes (peak.hip) ----------------
// kind 0: copy the first half of buf into the second half, iters times; kind 1: an MFMA loop of
// iters steps on every CU (buf: at least 2048 * 256 floats, written only in an impossible case).
// *work: bytes moved (0) or flops (1).
hipError_t launch_peak_probe(int kind, void* buf, size_t bytes, int iters, double* work, hipStream_t s);

// ---------------- post-step (post.hip) ----------------
hipError_t launch_lock_update(const int32_t* row_pos, int R, const float* conf, const float* kl, float eps,
                              float conf_min, uint8_t* force, hipStream_t s);
hipError_t launch_unmask(int32_t* tokens, const float* conf, const int32_t* argmax, int B, int S, int mask_id,
                         int lo, int hi, int n, hipStream_t s);
// tokens[b, i] = argmax[b, i] for masked i in [lo, hi) with force[b, i] == 1.
hipError_t launch_unmask_forced(int32_t* tokens, const uint8_t* force, const int32_t* argmax, int B, int S,
                                int mask_id, int lo, int hi, hipStream_t s);
// force[b][lo + o] = max(force, mark) for the offsets o of one dilated round (post.hip).
hipError_t launch_dus_mark(uint8_t* force, int B, int S, int lo, int block, int stride, int stride_prev, uint8_t mark,
                           hipStream_t s);

}  // namespace dllm
