// Host-side launchers of the LatentMoE HIP kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tokens per routing chunk: top-k records, per chunk and expert, a 32-bit
// mask of the chunk's tokens that picked the expert.
constexpr int kChunk = 32;
// Chunks per super-chunk of the two-level prefix sum.
constexpr int kSuper = 16;
// Token slices of the QB histogram kept in the state ([slice][E][B]).
constexpr int kHistSlices = 16;
// Rows per tile of the grouped expert GEMMs (also the granularity of the
// per-expert tile offsets computed by the scan).
#ifndef MOE_EXPERT_BM
#define MOE_EXPERT_BM 64
#endif
constexpr int kExpertBM = MOE_EXPERT_BM;
// Experts per block of the histogram kernel (16 x 256 bins = 16 KB of LDS).
constexpr int kHistExperts = 16;

struct Dims {
  int d, l, E, k, f, f_s, B;
  bool bf16;
  float eps, routed_scale;
};

hipError_t launch_rmsnorm(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s);
// Scores, biased top-k, gates and selection masks; with `hist` non-NULL
// (training) the same launch adds the score histogram and the token count.
hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       uint32_t* bitmap, uint32_t* hist, unsigned long long* count, hipStream_t s);
// Two launches: per-super-chunk prefix, then the global prefix, the row and
// m-tile offsets and the m-tile table tile_info[g] = {first row, expert << 8 |
// rows in use} of the grouped GEMMs.  With `load` non-NULL (sign-rule training) the
// counts are also added to load[E] and T to *count.
hipError_t launch_scan(const Dims& D, const uint32_t* bitmap, int T, int32_t* cbase, int32_t* sbase, int32_t* counts,
                       int32_t* offsets, int32_t* tile_offsets, int2* tile_info, uint32_t* load,
                       unsigned long long* count, hipStream_t s);
// Rows of the permutation, and the dispatch buffer X[row] = z[token].
// With zs non-NULL (MXFP8 experts) also copies each token's z scale row
// (s_ld bytes, a multiple of 4) to Xs at each of its grouped rows.
hipError_t launch_scatter(const Dims& D, const int32_t* idx, const uint32_t* bitmap, const int32_t* cbase,
                          const int32_t* sbase, int T, int32_t* perm_src, int32_t* inv, hipStream_t s,
                          const uint8_t* zs = nullptr, uint8_t* Xs = nullptr, int s_ld = 0);
hipError_t launch_combine(const Dims& D, const void* Y, const float* gates, const int32_t* inv, int T,
                          void* y_lat, hipStream_t s);
hipError_t launch_qb_quantile(const Dims& D, uint32_t* hist, const unsigned long long* count, double* q,
                              hipStream_t s);
hipError_t launch_qb_bias(const Dims& D, const double* q, unsigned long long* count, float* bias, hipStream_t s);
// Sign-rule bias update from the accumulated loads; clears loads and count.
hipError_t launch_sign_bias(const Dims& D, uint32_t* load, unsigned long long* count, float gamma, float* bias,
                            hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Dense GEMMs on h (router logits, shared GLU hidden, latent z) and for the
// output ([G | y_lat] [W_sd | W_up]^T).
// h [T,d] against [W_r | W_sg,W_su | W_dn] -> fp32 router logits (+ offset),
// shared GLU hidden G and latent z in one launch; a NULL output drops its
// part.
hipError_t launch_gemm_h(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                         const void* W_sg, const void* W_su, const void* W_dn, float* logits, void* G, void* z,
                         hipStream_t s);
// h against W_r alone -> fp32 logits (+ offset) (the routing-only pass).
hipError_t launch_gemm_rz(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                          float* logits, hipStream_t s);
hipError_t launch_gemm_out(const Dims& D, const void* G, const void* y_lat, int T, const void* W_sd,
                           const void* W_up, void* out, hipStream_t s);
// Grouped expert GEMMs over the rows grouped by expert (m-tiles of
// kExpertBM rows from tile_info; n_mtiles points at their count).
int expert_max_mtiles(int T, int k, int E);
// Expert GEMM 1 + GLU; its A rows are z[perm_src[r]] (the dispatch is part
// of the operand load, no dispatch buffer is written).
hipError_t launch_expert_up(const Dims& D, const void* z, const int32_t* perm_src, const int2* tile_info,
                            const int32_t* n_mtiles, int T, const void* W_g, const void* W_u, void* H, hipStream_t s);
hipError_t launch_expert_down(const Dims& D, const void* H, const int2* tile_info, const int32_t* n_mtiles, int T,
                              const void* W_d, void* Y, hipStream_t s);

// ---------------------------------------------------------------- backward --
// One column segment of a dense NT product C = A B^T: B [N, K] rows of ldb
// bytes; kind 0 = fp32 output, 1 = output in the activation dtype.
struct DenseSegSpec {
  const void* B;
  int N;
  int kind;
  void* out;
  int ldo;
};
// Dense C = A B^T, A [M, K] (lda bytes), up to 3 column segments sharing
// ldb; K_bytes a multiple of the stage row (128 B).  `tag` (3..7) only names
// the launch for profiles.
hipError_t launch_dense_nt(const Dims& D, int tag, const void* A, int lda_bytes, int M, int K_bytes,
                           const DenseSegSpec* segs, int nseg, int ldb_bytes, hipStream_t s);
// Grouped C_e = A_e W_e^T over the forward's expert m-tiles (rows grouped by
// expert, optionally gathered: A row of grouped row r = gather[r]); W_e at
// W + e * w_expert_bytes, [N, K]; output in the activation dtype.
hipError_t launch_expert_nt(const Dims& D, const void* A, int lda_bytes, const int32_t* gather, const void* W,
                            size_t w_expert_bytes, int ldb_bytes, int N, int K_bytes, const int2* tile_info,
                            const int32_t* n_mtiles, int T, void* out, int ldo, hipStream_t s);
// Per-expert fp32 C_e [M, N] = A_e B_e^T, K = pad_e = koff[e+1] - koff[e]:
// A_e is the block [M, pad_e] at element koff[e] * M of A, B_e [N, pad_e] at
// koff[e] * N of B (the segment layout of launch_transpose).
// With nseg > 0 and lda, ldb > 0 (elements) instead: nseg K slices
// koff[j] .. koff[j+1] of one product of row-major A [M, *] and B [N, *],
// partial C_j at out + j*M*N (split K).
hipError_t launch_wgrad(const Dims& D, const void* A, const void* B, const int32_t* koff, int M, int N, float* out,
                        hipStream_t s, int nseg = 0, long long lda = 0, long long ldb = 0);
// koff[j] = min(j * step, total) for j <= n (split-K boundaries).
hipError_t launch_fill_koff(int32_t* koff, int n, int step, int total, hipStream_t s);
// Sum of S fp32 partials [S, M, N] into up to 4 outputs, each a block of
// rows (by_rows) or of columns of C: segment i covers [start_i, start_i +
// len_i) and is stored row-major with ld_i at out_i.
struct SplitOut {
  int nseg, by_rows;
  int start[4], len[4], ld[4];
  float* out[4];
};
hipError_t launch_reduce_split(const float* part, int S, int M, int N, const SplitOut& o, hipStream_t s);

// dst[c][col_off + p] = src[gather[colmap[p]]][c] (maps optional), 0 for
// rows < 0 or >= R; `batch` matrices at the given strides (elements).  With
// seg_tile, expert e's columns seg_koff[e] .. seg_koff[e+1] go to their own
// contiguous block [C, pad_e] at element seg_koff[e] * C (ld_dst, col_off
// unused; C and P multiples of 64).
hipError_t launch_transpose(const Dims& D, const void* src, int R, int C, long long ld_src, long long src_bstride,
                            const int32_t* gather, const int32_t* colmap, int P, void* dst, long long ld_dst,
                            long long col_off, long long dst_bstride, int batch, hipStream_t s,
                            const int32_t* seg_koff = nullptr, const int32_t* seg_tile = nullptr);
// Padded per-expert K segments (whole 64-element stages, at least one) and
// the map from padded column to grouped row (-1 = pad) up to Kt columns.
hipError_t launch_pad_map(const Dims& D, const int32_t* offsets, int Kt, int32_t* koff, int32_t* colmap,
                          int32_t* seg_tile, hipStream_t s);
hipError_t launch_glu_bwd(const Dims& D, const void* P, const void* Q, const void* dG, long long R, int n, void* dP,
                          void* dQ, int ldo, hipStream_t s);
hipError_t launch_combine_bwd(const Dims& D, const void* dy, const void* Y, const float* gates, const int32_t* inv,
                              int T, void* dY, float* dg, hipStream_t s);
hipError_t launch_dispatch_bwd(const Dims& D, const void* dX, const int32_t* inv, int T, void* dz, int ldo,
                               hipStream_t s);
hipError_t launch_gates_bwd(const Dims& D, const float* logits, const int32_t* idx, const float* dg, int T, int Epad,
                            void* dl, int ldo, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const Dims& D, const void* x, const float* gamma, const float* dh, int T, void* dx,
                              float* rstd, float* part, int slices, float* dgamma, hipStream_t s);

// ------------------------------------------------------------------ MXFP8 --
// rows x K bf16 (ld_src elements) -> E4M3 bytes [rows, K] + E8M0 scales
// [rows, K/32] (one per 32 consecutive elements).
hipError_t launch_mx_quant(const void* src, long long rows, int K, long long ld_src, uint8_t* dst, uint8_t* scales,
                           hipStream_t s);
// Expert GEMM 1 + GLU with MXFP8 operands (A rows z8[perm_src[r]] with the
// scale rows Xs[r] the scatter copied; K = l <= 512, a multiple of 128); H
// in bf16.
hipError_t launch_expert_up_mx(const Dims& D, const uint8_t* z8, const uint8_t* Xs, const int32_t* perm_src,
                               const int2* tile_info, const int32_t* n_mtiles, int T, const uint8_t* Wg8,
                               const uint8_t* Wgs, const uint8_t* Wu8, const uint8_t* Wus, void* H, hipStream_t s);
// Expert GEMM 2 with MXFP8 operands (K = f <= 512, a multiple of 128); Y in bf16.
hipError_t launch_expert_down_mx(const Dims& D, const uint8_t* H8, const uint8_t* Hs, const int2* tile_info,
                                 const int32_t* n_mtiles, int T, const uint8_t* Wd8, const uint8_t* Wds, void* Y,
                                 hipStream_t s);

}  // namespace moe
