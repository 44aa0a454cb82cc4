/*
 * moe.h - C ABI of the Stable LatentMoE layer forward pass and its
 * quantile-balancing (QB) router-bias update on one AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (architecture paragraph and Tab 1 of the "Kimi K3 MoE lightweight
 * replica demo" article; design survival table of the Attention->K3 course,
 * Day 28):
 *   h     = RMSNorm(x)                    per token, gamma-scaled, eps = rms_eps
 *   l     = h W_r^T (+ c)                 router logits, fp32
 *   s     = sigmoid(l)                    scores (fp32, fixed op by op)
 *   idx   = top-k of s + b                the bias b only reroutes
 *   g     = s[idx] / sum s[idx]           gates, renormalised, bias-free
 *   G     = silu(h W_sg^T) * (h W_su^T)   shared expert at model width d
 *   z     = h W_dn^T                      down-projection to latent width l
 *   Y_e   = (silu(z W_g[e]^T) * (z W_u[e]^T)) W_d[e]^T   routed experts at l
 *   y_lat = sum_j g_j Y_{idx_j}           gate-weighted combine
 *   out   = G W_sd^T + y_lat W_up^T       no residual (the model adds its own)
 * QB (Tab 2 Fig. 2(b) and Tab 8-10 of the demo article; idle-experts section
 * of the "K3 tops open source" blog): every training forward adds each
 * token's score to a per-expert histogram; qb_update() turns the histogram
 * into the score q_e each expert must beat to get its share T*k/E of the
 * tokens and sets b_e = mean(q) - q_e (mean-centred); the new bias is used by
 * the next forward (one step late); in frozen mode nothing is accumulated or
 * updated.
 * Sign-rule balancer (capsule 16 of the "Pretraining a Mini Kimi K3" e-book
 * review, the noaux_tc bias rule), selected with moe_config.balancer: every
 * training forward adds each expert's token count to a per-expert load, and
 * the update moves each bias by sign_gamma towards balance:
 * b_e += sign_gamma * sign(mean load - load_e).
 *
 * Conventions
 *   - Every pointer argument named as device memory is a HIP device pointer
 *     the caller allocated; the library never allocates device memory and
 *     keeps no pointer past moe_destroy() other than those in moe_weights and
 *     the state buffer, which must outlive the context.
 *   - Weights are row-major [out, in] (y = x W^T).  In MOE_BF16 mode x, out
 *     and every weight except gamma and logit_offset are bf16; in MOE_F32 mode
 *     all are fp32.  Logits, scores, gates and the bias are fp32; indices are
 *     int32.  Accumulation is fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call that
 *     takes a stream only enqueues work on it and returns; results are valid
 *     once the stream has reached them.  No call synchronises the device or
 *     copies to the host, so forward/route/update can be captured in a graph.
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     a failed check returns an error code and enqueues nothing.  A launch
 *     failure returns MOE_ERR_HIP.  moe_last_error() gives a message for the
 *     last failure on the calling thread.  A context is not thread-safe.
 *   - Calls that share a context, or a workspace, must be ordered (one
 *     stream, or events) by the caller.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, unknown enum value            */
  MOE_ERR_SHAPE = 2,       /* sizes out of the supported ranges          */
  MOE_ERR_DTYPE = 3,       /* unsupported dtype                           */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  MOE_ERR_STATE = 5,       /* QB state would overflow; bad call order    */
  MOE_ERR_HIP = 6          /* a HIP runtime call or a launch failed      */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Tab 10 of the demo article: QB updates during training, frozen at inference. */
typedef enum moe_qb_mode { MOE_QB_TRAIN = 0, MOE_QB_FROZEN = 1 } moe_qb_mode;

/*
 * Which rule qb_update() applies.  MOE_BALANCE_QB: quantile balancing from
 * the score histogram (the demo article, Tab 8-10).  MOE_BALANCE_SIGN: the
 * sign rule of capsule 16 of the e-book review, b_e += sign_gamma *
 * sign(mean load - load_e) from the per-expert token counts (sign_gamma = 1e-2
 * there); the histogram is then neither built nor read.
 */
typedef enum moe_balancer { MOE_BALANCE_QB = 0, MOE_BALANCE_SIGN = 1 } moe_balancer;

/*
 * Storage of the routed experts' operands.  MOE_EXPERTS_BF16: as the rest of
 * the layer.  MOE_EXPERTS_MXFP8 (low-precision experts, bf16 mode only; l
 * and f multiples of 128, at most 512): W_g, W_u, W_d are held in the state
 * buffer as OCP MXFP8 -- FP8 E4M3 elements with one power-of-two E8M0 scale
 * per 32 consecutive elements along the contraction axis -- quantised at
 * moe_init (again by moe_requantize_experts after the caller changes them);
 * each forward quantises z and the expert hidden H the same way, and the
 * expert GEMMs multiply on the MFMA's block-scaled FP8 path with fp32 sums.
 * MOE_EXPERTS_MXFP4 (same conditions): 4-bit expert weights with 8-bit
 * activations ("K3 tops open source" blog, fourth-waste section; the format
 * is not named there, this is the OCP one): W_g, W_u, W_d as MXFP4 -- E2M1
 * elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two per byte,
 * low nibble first, with the same E8M0 scale per 32 along K, 2^(floor(log2
 * amax) - 2) -- against z and H in MXFP8 as above.
 * The backward pass needs MOE_EXPERTS_BF16.
 */
typedef enum moe_expert_format {
  MOE_EXPERTS_BF16 = 0,
  MOE_EXPERTS_MXFP8 = 1,
  MOE_EXPERTS_MXFP4 = 2
} moe_expert_format;

/*
 * Layer sizes.  d, l, f must be multiples of 64 and f_s a multiple of 64 or 0.
 * n_shared shared experts (>= 0), each a GLU of hidden f_s at width d (the
 * shared path of the demo article's architecture paragraph); their outputs
 * add, so they are held as one GLU of hidden n_shared*f_s: W_sg, W_su are
 * [n_shared*f_s, d] (expert i's hidden units at rows i*f_s ..) and W_sd is
 * [d, n_shared*f_s].  No shared path when n_shared*f_s == 0.
 * 1 <= E <= 1024, 1 <= k <= min(E, 32), 2 <= qb_bins <= 256.
 * qb_lo < qb_hi (finite): the QB histogram has qb_bins equal bins over the
 * score range [qb_lo, qb_hi] (Tab 2 Fig. 2(b) of the demo article: a
 * histogram estimate of each expert's score quantile); a score s falls in bin
 * clamp(floor(fp32(fp32(s - qb_lo) * scale)), 0, qb_bins - 1) with scale =
 * fp32(qb_bins / (qb_hi - qb_lo)) (quotient in fp64), so scores beyond the
 * range count in the end bins, and the quantile estimate is mapped back as
 * qb_lo + (qb_hi - qb_lo) * u (fp64).  Sigmoid scores lie in (0, 1): the
 * range [0, 1] covers them all; a narrower range that still holds every
 * expert's target quantile gives narrower bins.
 * max_tokens bounds T for every call (1 <= max_tokens, max_tokens*k < 2^31).
 * rms_eps > 0.  routed_scale multiplies every gate (1 = plain renormalised).
 * balancer picks the update rule; sign_gamma (finite, > 0) is read only for
 * MOE_BALANCE_SIGN.  A zero-filled tail (balancer 0) selects QB.
 * keep_preact (0 or 1; bf16 experts only): every forward also stores the
 * GLU pre-activations -- P = h W_sg^T, Q = h W_su^T of the shared expert and
 * A = X W_g^T, U = X W_u^T of the routed experts, in the activation dtype --
 * in the workspace (moe_ws_layout P, Q, A, U), and moe_backward reads them
 * instead of recomputing them (two GEMM passes fewer per training step, for
 * 2 (T f_s + T k f) more stored elements per forward).
 */
typedef struct moe_config {
  int32_t d, l, E, k, f, f_s, n_shared;
  moe_dtype dtype;
  float rms_eps;
  int32_t qb_bins;
  float qb_lo, qb_hi;
  moe_qb_mode qb_mode;
  int64_t max_tokens;
  float routed_scale;
  moe_balancer balancer;
  float sign_gamma;
  moe_expert_format experts;
  int32_t keep_preact;
} moe_config;

/* Device pointers, caller-owned, read-only to the library. */
typedef struct moe_weights {
  const float* gamma;        /* [d]     fp32 RMSNorm scale                 */
  const void* W_r;           /* [E,d]   router                             */
  const float* logit_offset; /* [E]     fp32 added to the logits, or NULL: a
                                learned router logit bias, which (unlike the
                                QB bias) also moves the scores and gates   */
  const void* W_sg;          /* [n_shared*f_s,d] shared gate (NULL: no shared path) */
  const void* W_su;          /* [n_shared*f_s,d] shared up                       */
  const void* W_sd;          /* [d,n_shared*f_s] shared down                     */
  const void* W_dn;          /* [l,d]   down-projection d -> l             */
  const void* W_g;           /* [E,f,l] expert gate                        */
  const void* W_u;           /* [E,f,l] expert up                          */
  const void* W_d;           /* [E,l,f] expert down                        */
  const void* W_up;          /* [d,l]   up-projection l -> d               */
} moe_weights;

/*
 * Routing results (device pointers).  Any field may be NULL; the library then
 * keeps that array in the workspace.  Rows of the permutation are grouped by
 * expert (offsets[e] .. offsets[e+1]) and keep token order inside a group.
 */
typedef struct moe_route_out {
  float* logits;     /* [T,E]  fp32 router logits                      */
  int32_t* topk_idx; /* [T,k]  experts by biased score desc, index asc */
  float* gates;      /* [T,k]  renormalised unbiased scores            */
  int32_t* counts;   /* [E]    tokens per expert                       */
  int32_t* offsets;  /* [E+1]  exclusive prefix sum of counts          */
  int32_t* perm_src; /* [T*k]  token of each grouped row               */
  int32_t* inv;      /* [T,k]  grouped row of each (token, slot)       */
} moe_route_out;

/* Byte offsets of the pieces of the QB state buffer (see moe_state_bytes). */
typedef struct moe_state_layout {
  size_t bias;  /* [E] fp32 router bias                                   */
  size_t count; /* uint64 tokens accumulated since the last qb_update     */
  size_t q;     /* [E] fp64 quantiles of the last qb_update               */
  size_t hist;  /* [hist_slices, E, qb_bins] uint32 score histogram (one
                   slice; the histogram is the sum over the slices)       */
  size_t hist_slices;
  size_t load;  /* [E] uint32 tokens routed to each expert since the last
                   update (sign-rule balancer only)                       */
  size_t mx;    /* block-scaled experts only: W_g, W_u [E,f,l] and W_d
                   [E,l,f] as E4M3 bytes (MXFP8) or E2M1 pairs [.., K/2]
                   (MXFP4), then their E8M0 scales [.., K/32]             */
  size_t total;
} moe_state_layout;

/* Byte offsets, inside the workspace, of the intermediates of one call. */
typedef struct moe_ws_layout {
  size_t h, logits, idx, gates, bitmap, cbase, sbase, counts, offsets, tile_offsets, perm_src, inv, tile_info;
  size_t G, z, X, H, Y, y_lat; /* X: zero bytes (the expert GEMM reads z[perm_src[r]]
                                  directly, so no dispatch buffer is written) */
  size_t z8, zs, Xs, H8, Hs;    /* block-scaled experts only (else zero bytes): z and H as
                                  E4M3 bytes and E8M0 scales; Xs the scale rows of
                                  the grouped rows */
  size_t P, Q, A, U;            /* keep_preact only (else zero bytes): the GLU
                                  pre-activations, P, Q [T, n_shared f_s], A, U [T k, f]
                                  (grouped rows, as H) */
  size_t total;
} moe_ws_layout;

typedef struct moe_ctx moe_ctx;

/* Bytes of the QB state buffer for `cfg` (0 when cfg is invalid). */
size_t moe_state_bytes(const moe_config* cfg);
moe_status moe_state_layout_of(const moe_config* cfg, moe_state_layout* out);

/* Bytes of workspace moe_forward / moe_route need for T tokens (0 if invalid). */
size_t moe_workspace_bytes(const moe_config* cfg, int64_t T);
moe_status moe_workspace_layout(const moe_config* cfg, int64_t T, moe_ws_layout* out);

/*
 * Create a context for `cfg` over the caller's weights and QB state buffer
 * (moe_state_bytes(cfg) bytes of device memory, 256-byte aligned).  Enqueues
 * on `stream` the clearing of the state: bias 0, histogram 0, count 0
 * (and, for block-scaled experts, the quantisation of the expert weights).
 * *out receives a host object freed by moe_destroy(); it owns one internal
 * stream (default priority) and five timing-free events on the current
 * device, used by moe_backward and released by moe_destroy().
 */
moe_status moe_init(const moe_config* cfg, const moe_weights* w, void* state, void* stream, moe_ctx** out);

/*
 * Routing only (RMSNorm, router, scores, QB histogram in training mode,
 * biased top-k, gates, counts, offsets, permutation) for T tokens of x[T,d].
 * When `logits` (device fp32 [T,E]) is not NULL it replaces the router output
 * and x is not read (x may be NULL): routing is then a pure function of the
 * logits and the bias, bit for bit.
 */
moe_status moe_route(moe_ctx* ctx, const void* x, const float* logits, int64_t T, moe_route_out* r,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Whole layer for T tokens: out[T,d] from x[T,d] (0 <= T <= max_tokens; T=0
 * enqueues nothing).  In training mode also adds the tokens' scores to the QB
 * histogram.  `r` (may be NULL) receives the routing.  `ws` must hold
 * moe_workspace_bytes(cfg, T) bytes of device memory (256-byte aligned).
 *
 * Statistics window.  The histogram bins and loads are 32-bit counters, so
 * one window (the training tokens between two qb_update calls) holds at
 * most 2^32 - 1 tokens.  A forward or routing call that would pass that
 * returns MOE_ERR_STATE before enqueueing anything; the host counts the
 * tokens of the calls it sees.  Replays of a captured graph are not calls:
 * a graph that holds training forwards should hold qb_update too (or be
 * replayed fewer than (2^32 - 1) / T times between updates).  If a replayed
 * window does pass the limit, the device's own 64-bit token count catches
 * it: that qb_update leaves the bias unchanged, writes NaN to every q_e of
 * the state (moe_state_layout.q) and clears the window.  Nothing is ever
 * silently wrapped.
 */
moe_status moe_forward(moe_ctx* ctx, const void* x, int64_t T, void* out, moe_route_out* r, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): moe_forward with the workspace
 * taken from a fixed array of MOE_NOALLOC_SCRATCH_BYTES (160 MiB: one
 * forward of the replica-shaped layer, d=1024, l=256, E=256, k=6, f=512,
 * f_s=2048, at 8192 tokens) that the library holds on each GPU it runs on
 * until the process ends.  Same arguments and results as moe_forward; the
 * caller still provides x, out and (optionally) r.  A T whose
 * moe_workspace_bytes(cfg, T) exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing; the array's device address is looked up by moe_init (and on the
 * first call on any other device).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, threads or
 * contexts without ordering between them) race, so order them.  The array
 * keeps the last call's intermediates; nothing a call reads from it has to
 * start at zero.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
moe_status moe_forward_noalloc(moe_ctx* ctx, const void* x, int64_t T, void* out, moe_route_out* r, void* stream);

/*
 * Bias update from the statistics accumulated since the last update, then
 * those statistics and the token count are cleared; the new bias is used by
 * the next forward.  MOE_BALANCE_QB: from the histogram, b_e = mean(q) - q_e;
 * keeps the bias when no token was accumulated.  MOE_BALANCE_SIGN: from the
 * loads n_e, b_e <- fp32(b_e + sign_gamma * sign(sum(n) - E * n_e)) (the sign
 * of mean load - n_e, taken exactly in integers; 0 leaves b_e unchanged, so no
 * accumulated token changes nothing).  A no-op returning MOE_OK in frozen mode.
 */
moe_status qb_update(moe_ctx* ctx, void* stream);

/*
 * Gradients of the layer (fp32, the shapes of moe_weights; every pointer is
 * device memory, overwritten, not accumulated).  W_sg, W_su, W_sd may be NULL
 * when there is no shared path (n_shared * f_s == 0).  The router bias gets
 * no gradient: it only reroutes (Tab 8-10 of the demo article), so a routing
 * decision is a constant of the backward.
 */
typedef struct moe_grads {
  float* gamma; /* [d]     */
  float* W_r;   /* [E,d]   */
  float* W_sg;  /* [n_shared*f_s,d] */
  float* W_su;  /* [n_shared*f_s,d] */
  float* W_sd;  /* [d,n_shared*f_s] */
  float* W_dn;  /* [l,d]   */
  float* W_g;   /* [E,f,l] */
  float* W_u;   /* [E,f,l] */
  float* W_d;   /* [E,l,f] */
  float* W_up;  /* [d,l]   */
} moe_grads;

/* Bytes of backward workspace for T tokens (0 if invalid). */
size_t moe_backward_workspace_bytes(const moe_config* cfg, int64_t T);

/*
 * Backward pass of the forward that moe_forward(ctx, x, T, ..., r, fwd_ws,
 * ...) last wrote into fwd_ws (same x, T and route outputs r, which may be
 * NULL as in the forward; fwd_ws must not have been reused since): from
 * dout[T,d] (activation dtype) writes dx[T,d] (activation dtype) and every
 * weight gradient in *g, for the scalar sum(out * dout).  The chain: output
 * projections, combine transpose (dY rows, gate gradients), grouped expert
 * GEMM transposes with the GLU derivative (pre-activations recomputed),
 * dispatch transpose (sum of each token's k rows), gate renormalisation and
 * sigmoid derivative to the router logits, shared GLU, the summed gradient of
 * h, RMSNorm.  Weight gradients of the experts take each expert's own tokens
 * as the K range of one grouped product.  `ws` holds
 * moe_backward_workspace_bytes(cfg, T) bytes (256-byte aligned).  QB state
 * is neither read nor changed.  T = 0 enqueues nothing.  With keep_preact
 * the weight-gradient products run on the context's internal stream, forked
 * from `stream` by events after their operands are written and joined back
 * before the call returns (also when it returns an error after the fork),
 * so every result is still ordered on `stream` (and the call can still be
 * captured in a graph on `stream`); concurrent moe_backward calls on one
 * context are not allowed.
 */
moe_status moe_backward(moe_ctx* ctx, const void* x, const void* dout, int64_t T, const moe_route_out* r,
                        const void* fwd_ws, size_t fwd_ws_bytes, void* dx, const moe_grads* g, void* ws,
                        size_t ws_bytes, void* stream);

/* MXFP8 experts: quantise the caller's W_g, W_u, W_d again (after an update). */
moe_status moe_requantize_experts(moe_ctx* ctx, void* stream);

/* Copy the current bias (E fp32) to / from device memory on `stream`. */
moe_status moe_get_bias(moe_ctx* ctx, float* dst, void* stream);
moe_status moe_set_bias(moe_ctx* ctx, const float* src, void* stream);

/*
 * Self-check of the routing kernels' shortcut.  To skip work, the top-k and
 * histogram kernels first evaluate a fast router score (the same clamp, then
 * the hardware exp2 and reciprocal) and compute the exact score of the
 * "Stable LatentMoE" routing section (the specified sigmoid above) only where
 * a decision could depend on it; each such decision keeps at least twice
 * MOE_FAST_SCORE_ERR of room, so routing and histogram stay bit-identical to
 * the exact definition while every fp32 logit gives |fast - exact| <=
 * MOE_FAST_SCORE_ERR.  This call measures that difference on the device over
 * all 2^32 fp32 bit patterns and writes the largest one to err[0] (one float
 * of caller-owned device memory, overwritten).  Two launches on `stream`,
 * about 10 ms; nothing is allocated.  MOE_ERR_INVALID_ARG for a NULL err,
 * MOE_ERR_HIP if a launch fails.
 */
#define MOE_FAST_SCORE_ERR 0x1p-20f
moe_status moe_fast_score_error(float* err, void* stream);

/* Switch between training and frozen QB; the accumulated statistics are kept. */
moe_status moe_set_qb_mode(moe_ctx* ctx, moe_qb_mode mode);

void moe_destroy(moe_ctx* ctx);

const char* moe_status_string(moe_status s);
const char* moe_last_error(void);

/*
 * Per-kernel timing.  After moe_profile_begin(ctx, n, mask), each kernel the
 * context launches whose id has its bit set in `mask` (0 = every kernel), up
 * to n launches, is bracketed by HIP events on its stream.  moe_profile_end()
 * waits for those events and fills, for each kernel id 0..n_ids-1, the summed
 * milliseconds and the launch count; then profiling stops.  Host-side event
 * objects only; no device memory.  MOE_K_HIST, MOE_K_QB_BIAS and
 * MOE_K_BWD_TRANSPOSE are kept for numbering only and record no launches: in
 * training mode the QB histogram is built inside the MOE_K_TOPK launch, the
 * bias launch is timed with the quantile launch under MOE_K_QB_UPDATE, and
 * the backward's GEMMs read their operands as stored (K-major tiles), with
 * no transposed copies.
 */
enum {
  MOE_K_RMSNORM = 0, MOE_K_GEMM_H, MOE_K_TOPK, MOE_K_HIST, MOE_K_SCAN, MOE_K_SCATTER,
  MOE_K_EXPERT_UP, MOE_K_EXPERT_DOWN, MOE_K_COMBINE, MOE_K_GEMM_OUT,
  MOE_K_QB_UPDATE, /* the update's two launches: quantiles per expert, then mean and bias */
  MOE_K_QB_BIAS,   /* (numbering only: both launches are timed under MOE_K_QB_UPDATE) */
  MOE_K_GEMM_RZ, MOE_K_SIGN_BIAS,
  /* backward: dense products, grouped expert products, weight gradients,
     elementwise transposes and derivatives, (unused) */
  MOE_K_BWD_GEMM, MOE_K_BWD_EXPERT, MOE_K_BWD_WGRAD, MOE_K_BWD_ELTWISE, MOE_K_BWD_TRANSPOSE,
  MOE_K_MX_QUANT, /* MXFP8 quantisation of z (H is quantised in expert_up's epilogue) */
  MOE_NUM_KERNELS
};
const char* moe_kernel_name(int id);
moe_status moe_profile_begin(moe_ctx* ctx, int max_launches, uint32_t mask);
moe_status moe_profile_end(moe_ctx* ctx, double* ms, int64_t* launches, int n);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
