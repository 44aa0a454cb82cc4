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
// Token parts of one training pass whose score histograms are built by
// separate blocks (each adds its counts into the one histogram of the state),
// per 1024 threads of a top-k block (twice as many with 512-thread blocks,
// half as many in the 64-lane layout).
constexpr int kHistParts = 16;
// Rows per tile of the grouped expert GEMMs (also the granularity of the
// per-expert tile offsets computed by the scan).
#ifndef MOE_EXPERT_BM
#define MOE_EXPERT_BM 64
#endif
constexpr int kExpertBM = MOE_EXPERT_BM;
// Rows per tile of the second (coarser) tile table, used by the bf16 expert
// down-projection: its output is only l wide, so 64-row tiles leave 1.7
// waves of tiles on the chip at the replica shape and twice the weight passes.
constexpr int kExpertBM2 = 2 * kExpertBM;
// Experts per block of the histogram kernel (16 x 256 bins = 16 KB of LDS).
constexpr int kHistExperts = 16;

struct Dims {
  int d, l, E, k, f, f_s, B;  // f_s: hidden of the whole shared path (n_shared GLUs as one)
  bool bf16;
  float eps, routed_scale;
  float qb_lo, qb_hi, qb_scale;  // histogram score range and fp32(B / (qb_hi - qb_lo))
};

// The largest |fast - exact| router score difference over all 2^32 fp32
// logits, written (as a float) to out[0] on the device.
hipError_t launch_fast_score_error(float* out, hipStream_t s);
// RMSNorm; the launch also clears zero[0 .. nzero) (the super-chunk
// selection counts the top-k launch of the same pass adds into).
hipError_t launch_rmsnorm(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s,
                          int32_t* zero = nullptr, int nzero = 0);
// Scores, biased top-k, gates and selection masks, and each super-chunk's
// selection count per expert added to ssum[T / (kChunk kSuper)][E] (cleared
// beforehand); with `hist` non-NULL (training) the same launch adds the
// score histogram and the token count.
hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       uint32_t* bitmap, uint32_t* hist, unsigned long long* count, int32_t* ssum, hipStream_t s);
// The global prefix over the super-chunk totals sbase (which become each
// super-chunk's first row per expert), the row and m-tile offsets and the
// m-tile table tile_info[g] = {first row, expert << 8 | rows in use} of the
// grouped GEMMs.  With `load` non-NULL (sign-rule training) the counts are
// also added to load[E] and T to *count.
// tile_offsets / tile_info: the kExpertBM table; tile_offsets2 / tile_info2
// (nullable): the kExpertBM2 table.  The scan writes the tile tables only with
// at most 8 tiles per expert on average; otherwise the scatter launch does.
hipError_t launch_scan(const Dims& D, int T, int32_t* sbase, int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                       int2* tile_info, uint32_t* load, unsigned long long* count, hipStream_t s,
                       int32_t* tile_offsets2 = nullptr, int2* tile_info2 = nullptr);
// Rows of the permutation (perm_src, inv).  With zs non-NULL (MXFP8 experts)
// also copies each token's z scale row (s_ld bytes, a multiple of 4) to Xs at
// each of its grouped rows.  With many tiles per expert (more than 8 on
// average) the same launch writes the grouped GEMMs' tile tables from the
// scan's counts, offsets and tile offsets (tile_offsets2 / tile_info2 may be
// NULL); otherwise the scan has written them.
hipError_t launch_scatter(const Dims& D, const int32_t* idx, const uint32_t* bitmap, const int32_t* sbase, int T,
                          int32_t* perm_src, int32_t* inv, hipStream_t s, const uint8_t* zs, uint8_t* Xs, int s_ld,
                          const int32_t* counts, const int32_t* offsets, const int32_t* tile_offsets,
                          int2* tile_info, const int32_t* tile_offsets2, int2* tile_info2);
hipError_t launch_combine(const Dims& D, const void* Y, const float* gates, const int32_t* inv, int T,
                          void* y_lat, hipStream_t s);
// QB update: quantiles from the histogram [E][B] (cleared; one block per
// expert), then b = mean(q) - q and the token count cleared (one block).
hipError_t launch_qb_update(const Dims& D, uint32_t* hist, unsigned long long* count, double* q, float* bias,
                            hipStream_t s);
// Sign-rule bias update from the accumulated loads; clears loads and count.
hipError_t launch_sign_bias(const Dims& D, uint32_t* load, unsigned long long* count, float gamma, float* bias,
                            hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Dense GEMMs on h (router logits, shared GLU hidden, latent z) and for the
// output ([G | y_lat] [W_sd | W_up]^T).
// h [T,d] against [W_r | W_sg,W_su | W_dn] -> fp32 router logits (+ offset),
// shared GLU hidden G and latent z in one launch; a NULL output drops its
// part.  P, Q (both or neither): the GLU's pre-activations h W_sg^T, h W_su^T
// are stored there as well.
hipError_t launch_gemm_h(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                         const void* W_sg, const void* W_su, const void* W_dn, float* logits, void* G, void* z,
                         hipStream_t s, void* P = nullptr, void* Q = nullptr);
// h against W_r alone -> fp32 logits (+ offset) (the routing-only pass).
hipError_t launch_gemm_rz(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                          float* logits, hipStream_t s);
hipError_t launch_gemm_out(const Dims& D, const void* G, const void* y_lat, int T, const void* W_sd,
                           const void* W_up, void* out, hipStream_t s);
// Grouped expert GEMMs over the rows grouped by expert (m-tiles of
// kExpertBM rows from tile_info; n_mtiles points at their count).
int expert_max_mtiles(int T, int k, int E, int bm = kExpertBM);
// Expert GEMM 1 + GLU; its A rows are z[perm_src[r]] (the dispatch is part
// of the operand load, no dispatch buffer is written).  A, U (both or
// neither): the pre-activations X W_g^T, X W_u^T are stored there as well.
// tall: the tile table is the kExpertBM2-row one (many rows per expert).
hipError_t launch_expert_up(const Dims& D, const void* z, const int32_t* perm_src, const int2* tile_info,
                            const int32_t* n_mtiles, int T, const void* W_g, const void* W_u, void* H, hipStream_t s,
                            void* A = nullptr, void* U = nullptr, bool tall = false);
// Expert GEMM 2 over the kExpertBM2-row tile table (tile_info2, n_mtiles2).
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
// ldb; K_bytes a multiple of the stage row (128 B).  `tag` (3) only names
// the launch for profiles.
hipError_t launch_dense_nt(const Dims& D, int tag, const void* A, int lda_bytes, int M, int K_bytes,
                           const DenseSegSpec* segs, int nseg, int ldb_bytes, hipStream_t s);
// Grouped C_e = A_e W_e^T over the forward's expert m-tiles (rows grouped by
// expert, optionally gathered: A row of grouped row r = gather[r]); W_e at
// W + e * w_expert_bytes, [N, K]; output in the activation dtype.
hipError_t launch_expert_nt(const Dims& D, const void* A, int lda_bytes, const int32_t* gather, const void* W,
                            size_t w_expert_bytes, int ldb_bytes, int N, int K_bytes, const int2* tile_info,
                            const int32_t* n_mtiles, int T, void* out, int ldo, hipStream_t s);
// Weight gradients C_e = A_e^T B_e over segments e of the token axis, A and
// B token-major (no transposed copies): segment e is rows [koff[e],
// koff[e+1]) (koff null: [e kstep, (e+1) kstep)) cut at kend; B's columns
// n < nsplit come from B0 (row stride ldb0), the rest from B1; with gather,
// B's row k is row gather[k] of B0/B1 (gather has ngather entries).  Strides
// and nsplit in elements, multiples of 16 bytes; C_e [M, N] fp32 at out + e M N.
struct WgradKmSpec {
  const void* A;
  long long lda;
  const void* B0;
  long long ldb0;
  const void* B1;
  long long ldb1;
  int nsplit;
  const int32_t* koff;
  int kstep, kend;
  const int32_t* gather;
  int ngather;
  int M, N, nseg;
  float* out;
};
hipError_t launch_wgrad_km(const Dims& D, const WgradKmSpec& w, hipStream_t s);
// Data gradients C = A B with B K-major (weights as stored, read along their
// input index).  K is a concatenation of up to 4 pieces: piece j spans `span`
// K values (a multiple of 64) read from rows 0 .. rows-1 of B (row stride ldb
// elements, a multiple of 16 bytes); rows rows .. span-1 count as zero.  A is
// row-major with K contiguous (lda_bytes per row, the pieces' spans summed).
struct KPiece {
  const void* B;
  long long ldb;
  int span, rows;
};
struct DgradSegSpec {
  KPiece piece[4];
  int N, kind;  // kind 0: fp32 output, 1: output in the activation dtype
  void* out;
  int ldo;
};
// Dense: rows 0..M-1 of A, up to 2 output segments (same K pieces' spans and
// rows, each its own sources); tag 4 or 5 names the launch in profiles.
hipError_t launch_dgrad_dense(const Dims& D, int tag, const void* A, int lda_bytes, int M, const DgradSegSpec* segs,
                              int nseg, int npiece, hipStream_t s);
// Grouped expert rows (tiles of the dispatch order), B advancing by
// b_expert_bytes per expert; output in the activation dtype; tag 8 or 9.
hipError_t launch_dgrad_expert(const Dims& D, int tag, const void* A, int lda_bytes, const KPiece* pieces, int npiece,
                               size_t b_expert_bytes, int N, const int2* tile_info, const int32_t* n_mtiles, int T,
                               void* out, int ldo, hipStream_t s);
// Sum of S fp32 partials [S, M, N] into up to 4 outputs, each a block of
// rows (by_rows) or of columns of C: segment i covers [start_i, start_i +
// len_i) and is stored row-major with ld_i at out_i.
struct SplitOut {
  int nseg, by_rows;
  int start[4], len[4], ld[4];
  float* out[4];
};
hipError_t launch_reduce_split(const float* part, int S, int M, int N, const SplitOut& o, hipStream_t s);

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

// ------------------------------------------------------- block-scaled experts --
// rows x K bf16 (ld_src elements) -> E4M3 bytes [rows, K] + E8M0 scales
// [rows, K/32] (one per 32 consecutive elements); w4: E2M1 elements two per
// byte (low nibble first) [rows, K/2] with the MXFP4 scale instead.
hipError_t launch_mx_quant(const void* src, long long rows, int K, long long ld_src, uint8_t* dst, uint8_t* scales,
                           hipStream_t s, bool w4 = false);
// Expert GEMM 1 + GLU with MXFP8 activations (A rows z8[perm_src[r]] with the
// scale rows Xs[r] the scatter copied; K = l <= 512, a multiple of 128) and
// MXFP8 weights, or MXFP4 weights with w4; H in bf16, and H quantised to
// MXFP8 in the epilogue (H8 [rows, f] bytes, Hs [rows, f/32] scales).
hipError_t launch_expert_up_mx(const Dims& D, const uint8_t* z8, const uint8_t* Xs, const int32_t* perm_src,
                               const int2* tile_info, const int32_t* n_mtiles, int T, const uint8_t* Wg8,
                               const uint8_t* Wgs, const uint8_t* Wu8, const uint8_t* Wus, void* H, uint8_t* H8,
                               uint8_t* Hs, hipStream_t s, bool w4 = false);
// Expert GEMM 2 with MXFP8 activations (K = f <= 512, a multiple of 128) and
// MXFP8 or (w4) MXFP4 weights; Y in bf16.
hipError_t launch_expert_down_mx(const Dims& D, const uint8_t* H8, const uint8_t* Hs, const int2* tile_info,
                                 const int32_t* n_mtiles, int T, const uint8_t* Wd8, const uint8_t* Wds, void* Y,
                                 hipStream_t s, bool w4 = false);

}  // namespace moe
