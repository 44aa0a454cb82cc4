// C ABI of the LatentMoE layer (include/moe.h): argument checks, workspace
// and state layouts, the launch sequence of a forward / routing pass / QB
// update, and optional per-kernel event timing.  Host code only; all device
// memory belongs to the caller.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"

using namespace moe;

// Workspace of moe_forward_noalloc: one array per GPU, in the library's code
// object, so that forward needs no allocation.  Each GPU the library's kernels
// are loaded on holds it until the process ends.  In host code the name is a
// host-side stand-in, never the device memory: kernels and copies only ever
// get the device address that hipGetSymbolAddress returns for it.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Hidden width of the shared path: n_shared GLUs of hidden f_s held as one.
int32_t shared_hidden(const moe_config* c) { return c->n_shared * c->f_s; }

// Bins per unit of score: fp32(B / (hi - lo)), the quotient in fp64.
float qb_scale(const moe_config* c) {
  return (float)((double)c->qb_bins / ((double)c->qb_hi - (double)c->qb_lo));
}

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "unknown dtype %d", (int)c->dtype);
  if (c->qb_mode != MOE_QB_TRAIN && c->qb_mode != MOE_QB_FROZEN)
    return fail(MOE_ERR_INVALID_ARG, "unknown qb_mode %d", (int)c->qb_mode);
  if (c->balancer != MOE_BALANCE_QB && c->balancer != MOE_BALANCE_SIGN)
    return fail(MOE_ERR_INVALID_ARG, "unknown balancer %d", (int)c->balancer);
  if (c->balancer == MOE_BALANCE_SIGN && !(c->sign_gamma > 0.f && std::isfinite(c->sign_gamma)))
    return fail(MOE_ERR_INVALID_ARG, "sign_gamma must be finite and > 0");
  if (c->experts != MOE_EXPERTS_BF16 && c->experts != MOE_EXPERTS_MXFP8 && c->experts != MOE_EXPERTS_MXFP4)
    return fail(MOE_ERR_INVALID_ARG, "unknown expert format %d", (int)c->experts);
  if (c->experts != MOE_EXPERTS_BF16) {
    const char* fmt = c->experts == MOE_EXPERTS_MXFP8 ? "MXFP8" : "MXFP4";
    if (c->dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "%s experts need the bf16 mode", fmt);
    if (c->l % 128 || c->f % 128 || c->l > 512 || c->f > 512)
      return fail(MOE_ERR_SHAPE, "%s experts need l and f multiples of 128, at most 512 (l=%d f=%d)", fmt, c->l,
                  c->f);
  }
  if (c->keep_preact != 0 && c->keep_preact != 1) return fail(MOE_ERR_INVALID_ARG, "keep_preact must be 0 or 1");
  if (c->keep_preact && c->experts != MOE_EXPERTS_BF16)
    return fail(MOE_ERR_INVALID_ARG, "keep_preact needs bf16 experts");
  auto m64 = [](int32_t v) { return v > 0 && v % 64 == 0; };
  if (!m64(c->d) || !m64(c->l) || !m64(c->f))
    return fail(MOE_ERR_SHAPE, "d, l, f must be positive multiples of 64 (d=%d l=%d f=%d)", c->d, c->l, c->f);
  if (c->f_s < 0 || c->f_s % 64 != 0) return fail(MOE_ERR_SHAPE, "f_s must be 0 or a multiple of 64 (f_s=%d)", c->f_s);
  if (c->n_shared < 0) return fail(MOE_ERR_SHAPE, "n_shared must be >= 0 (n_shared=%d)", c->n_shared);
  if (c->d > (1 << 20) || c->l > (1 << 20) || c->f > (1 << 20) || (int64_t)c->n_shared * c->f_s > (1 << 20))
    return fail(MOE_ERR_SHAPE, "a width (or n_shared*f_s) exceeds 2^20");
  if (!std::isfinite(c->qb_lo) || !std::isfinite(c->qb_hi) || !(c->qb_lo < c->qb_hi))
    return fail(MOE_ERR_INVALID_ARG, "the histogram range needs finite qb_lo < qb_hi (%g, %g)", (double)c->qb_lo,
                (double)c->qb_hi);
  if (!std::isfinite(qb_scale(c)))
    return fail(MOE_ERR_INVALID_ARG, "qb_bins / (qb_hi - qb_lo) overflows fp32");
  if (c->E < 1 || c->E > 1024) return fail(MOE_ERR_SHAPE, "E must be in [1, 1024] (E=%d)", c->E);
  if (c->k < 1 || c->k > 32 || c->k > c->E) return fail(MOE_ERR_SHAPE, "k must be in [1, min(E, 32)] (k=%d)", c->k);
  if (c->qb_bins < 2 || c->qb_bins > 256) return fail(MOE_ERR_SHAPE, "qb_bins must be in [2, 256] (%d)", c->qb_bins);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be > 0");
  if (!std::isfinite(c->routed_scale)) return fail(MOE_ERR_INVALID_ARG, "routed_scale must be finite");
  if (c->max_tokens < 1 || c->max_tokens * (int64_t)c->k >= (int64_t(1) << 31))
    return fail(MOE_ERR_SHAPE, "max_tokens must be >= 1 with max_tokens*k < 2^31");
  return MOE_OK;
}

Dims dims_of(const moe_config* c) {
  Dims D;
  D.d = c->d;
  D.l = c->l;
  D.E = c->E;
  D.k = c->k;
  D.f = c->f;
  D.f_s = shared_hidden(c);
  D.B = c->qb_bins;
  D.bf16 = c->dtype == MOE_BF16;
  D.eps = c->rms_eps;
  D.routed_scale = c->routed_scale;
  D.qb_lo = c->qb_lo;
  D.qb_hi = c->qb_hi;
  D.qb_scale = qb_scale(c);
  return D;
}

void state_layout(const moe_config* c, moe_state_layout* L) {
  size_t o = 0;
  L->bias = o;
  o = up(o + (size_t)c->E * 4);
  L->count = o;
  o = up(o + 8);
  L->q = o;
  o = up(o + (size_t)c->E * 8);
  L->hist = o;
  L->hist_slices = 1;
  o = up(o + (size_t)c->E * c->qb_bins * 4);
  L->load = o;
  o = up(o + (size_t)c->E * 4);
  L->mx = o;
  if (c->experts != MOE_EXPERTS_BF16) {
    const size_t w = (size_t)c->E * c->f * c->l;  // elements of each expert weight tensor
    const size_t wb = c->experts == MOE_EXPERTS_MXFP4 ? w / 2 : w;  // their bytes: E2M1 pairs or E4M3
    o = up(o + 3 * wb + 3 * (w / 32));
  }
  L->total = o;
}

void ws_layout(const moe_config* c, int64_t T, moe_ws_layout* L) {
  const size_t es = c->dtype == MOE_BF16 ? 2 : 4;
  const size_t t = (size_t)T, E = (size_t)c->E, k = (size_t)c->k;
  const size_t nchunks = (t + kChunk - 1) / kChunk;
  const size_t nsuper = (nchunks + kSuper - 1) / kSuper;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes);
    return at;
  };
  L->h = take(t * c->d * es);
  L->logits = take(t * E * 4);
  L->idx = take(t * k * 4);
  L->gates = take(t * k * 4);
  L->bitmap = take(nchunks * E * 4);
  L->cbase = take(0);  // kept in the layout, no longer used (the scatter sums chunk bases from the masks)
  L->sbase = take(nsuper * E * 4);
  L->counts = take(E * 4);
  L->offsets = take((E + 1) * 4);
  L->tile_offsets = take(2 * (E + 1) * 4);  // the kExpertBM table's, then the kExpertBM2 table's
  L->perm_src = take(t * k * 4);
  L->inv = take(t * k * 4);
  L->tile_info = take(T > 0 ? ((size_t)expert_max_mtiles((int)T, c->k, c->E) +
                                (size_t)expert_max_mtiles((int)T, c->k, c->E, kExpertBM2)) * 8
                             : 0);  // both tile tables
  const size_t fs = (size_t)shared_hidden(c);
  L->G = take(t * fs * es);
  L->z = take(t * c->l * es);
  L->X = take(0);  // no dispatch buffer: expert_up gathers z rows itself
  L->H = take(t * k * c->f * es);
  L->Y = take(t * k * c->l * es);
  L->y_lat = take(t * c->l * es);
  const bool mx = c->experts != MOE_EXPERTS_BF16;  // MXFP8 activations in both block-scaled formats
  L->z8 = take(mx ? t * c->l : 0);
  L->zs = take(mx ? t * c->l / 32 : 0);
  L->Xs = take(mx ? t * k * c->l / 32 : 0);
  L->H8 = take(mx ? t * k * c->f : 0);
  L->Hs = take(mx ? t * k * c->f / 32 : 0);
  const bool keep = c->keep_preact != 0;
  L->P = take(keep ? t * fs * es : 0);
  L->Q = take(keep ? t * fs * es : 0);
  L->A = take(keep ? t * k * c->f * es : 0);
  L->U = take(keep ? t * k * c->f * es : 0);
  L->total = o;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device address of `scratch` on each GPU, looked up once per device (with
// that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_HIP, "device %d: only %d devices are tracked", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress of the no-alloc scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

struct moe_ctx {
  moe_config cfg;
  moe_weights w;
  char* state;
  moe_state_layout sl;
  Dims D;
  uint64_t pending_tokens;  // accumulated into the histogram since the last update (host mirror)
  // per-kernel timing
  bool prof = false;
  uint32_t prof_mask = 0;
  int prof_max = 0, prof_n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int> ev_kernel;
  // backward: an internal stream for the weight-gradient products, forked
  // from and joined back to the caller's stream with these events
  hipStream_t side = nullptr;
  hipEvent_t fork_ev[4] = {}, join_ev = nullptr;
};

namespace {

template <class F>
moe_status run(moe_ctx* c, int kid, hipStream_t s, F&& f) {
  const bool rec = c->prof && c->prof_n < c->prof_max && (c->prof_mask == 0 || ((c->prof_mask >> kid) & 1u));
  if (rec && hipEventRecord(c->ev[2 * c->prof_n], s) != hipSuccess)
    return fail(MOE_ERR_HIP, "hipEventRecord failed");
  hipError_t e = f();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch of %s failed: %s", moe_kernel_name(kid), hipGetErrorString(e));
  if (rec) {
    if (hipEventRecord(c->ev[2 * c->prof_n + 1], s) != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord failed");
    c->ev_kernel[c->prof_n++] = kid;
  }
  return MOE_OK;
}

#define MOE_RUN(kid, expr)                                         \
  do {                                                             \
    moe_status st_ = run(ctx, kid, s, [&]() { return (expr); }); \
    if (st_ != MOE_OK) return st_;                                 \
  } while (0)

struct RoutePtrs {
  float* logits;
  int32_t *idx, *sbase, *counts, *offsets, *tile_offsets, *perm_src, *inv;
  int nsbase;  // ints in sbase
  uint32_t* bitmap;
  int2* tile_info;
  int32_t* tile_offsets2;  // the kExpertBM2 tile table (expert down-projection)
  int2* tile_info2;
  float* gates;
};

RoutePtrs route_ptrs(const moe_config& c, int64_t T, const moe_ws_layout& L, char* ws, const moe_route_out* r) {
  RoutePtrs p;
  p.logits = (r && r->logits) ? r->logits : reinterpret_cast<float*>(ws + L.logits);
  p.idx = (r && r->topk_idx) ? r->topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  p.gates = (r && r->gates) ? r->gates : reinterpret_cast<float*>(ws + L.gates);
  p.counts = (r && r->counts) ? r->counts : reinterpret_cast<int32_t*>(ws + L.counts);
  p.offsets = (r && r->offsets) ? r->offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  p.perm_src = (r && r->perm_src) ? r->perm_src : reinterpret_cast<int32_t*>(ws + L.perm_src);
  p.inv = (r && r->inv) ? r->inv : reinterpret_cast<int32_t*>(ws + L.inv);
  p.bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  p.sbase = reinterpret_cast<int32_t*>(ws + L.sbase);
  p.nsbase = (int)((((T + kChunk - 1) / kChunk + kSuper - 1) / kSuper) * c.E);
  p.tile_offsets = reinterpret_cast<int32_t*>(ws + L.tile_offsets);
  p.tile_info = reinterpret_cast<int2*>(ws + L.tile_info);
  p.tile_offsets2 = p.tile_offsets + (c.E + 1);
  p.tile_info2 = p.tile_info + (T > 0 ? expert_max_mtiles((int)T, c.k, c.E) : 0);
  return p;
}

// Checks of a call on T tokens with a workspace.  `accumulates`: the call
// adds T tokens to the training statistics (a forward or routing pass in
// training mode), so the window limit applies; the host counts the tokens of
// the calls it sees (a replayed graph is checked by the update kernels).
moe_status check_call(moe_ctx* ctx, int64_t T, void* ws, size_t ws_bytes, bool accumulates = true) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (T < 0 || T > ctx->cfg.max_tokens)
    return fail(MOE_ERR_SHAPE, "T=%lld outside [0, max_tokens=%lld]", (long long)T, (long long)ctx->cfg.max_tokens);
  if (T == 0) return MOE_OK;
  const size_t need = moe_workspace_bytes(&ctx->cfg, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (accumulates && ctx->cfg.qb_mode == MOE_QB_TRAIN && ctx->pending_tokens + (uint64_t)T >= (uint64_t(1) << 32))
    return fail(MOE_ERR_STATE, "more than 2^32-1 tokens accumulated without qb_update");
  return MOE_OK;
}

// Steps after the logits: scores, QB histogram, top-k + gates + selection
// masks, two-level prefix sums with offsets, stable rows (perm_src, inv).
moe_status route_tail(moe_ctx* ctx, const RoutePtrs& p, int T, hipStream_t s, const uint8_t* zs = nullptr,
                      uint8_t* Xs = nullptr) {
  const Dims& D = ctx->D;
  const float* bias = reinterpret_cast<const float*>(ctx->state + ctx->sl.bias);
  const bool train = ctx->cfg.qb_mode == MOE_QB_TRAIN;
  const bool sign = ctx->cfg.balancer == MOE_BALANCE_SIGN;
  // training statistics: the score histogram (QB) or the per-expert loads (sign rule)
  uint32_t* hist = train && !sign ? reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.hist) : nullptr;
  uint32_t* load = train && sign ? reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.load) : nullptr;
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(ctx->state + ctx->sl.count);
  MOE_RUN(MOE_K_TOPK, launch_topk(D, p.logits, bias, T, p.idx, p.gates, p.bitmap, hist, cnt, p.sbase, s));
  if (train) ctx->pending_tokens += (uint64_t)T;
  MOE_RUN(MOE_K_SCAN, launch_scan(D, T, p.sbase, p.counts, p.offsets, p.tile_offsets,
                                  p.tile_info, load, train && sign ? cnt : nullptr, s, p.tile_offsets2,
                                  p.tile_info2));
  MOE_RUN(MOE_K_SCATTER, launch_scatter(D, p.idx, p.bitmap, p.sbase, T, p.perm_src, p.inv, s, zs, Xs, D.l / 32,
                                        p.counts, p.offsets, p.tile_offsets, p.tile_info, p.tile_offsets2,
                                        p.tile_info2));
  return MOE_OK;
}

// ----------------------------------------------------------------- backward --
struct BwdLayout {
  size_t P, Q, dG, dy, dAcat, dg, dY, dH, Apre, U, dAU, dX, dh, rstd, gpart;
  size_t dWcat, total;
  int Tp, Epad, Kc;
};
constexpr int kGammaSlices = 64;
constexpr int kSplitOut = 3, kSplitCat = 3;  // K slices of the two dense weight-gradient products (144 and 304 output tiles at the replica shape: 3 slices fill 512 block slots best)

void bwd_layout(const moe_config* c, int64_t T, BwdLayout* L) {
  const size_t es = c->dtype == MOE_BF16 ? 2 : 4;
  const size_t t = (size_t)T, E = (size_t)c->E, k = (size_t)c->k, d = c->d, l = c->l, f = c->f,
               fs = (size_t)shared_hidden(c);
  const size_t Tk = t * k;
  L->Tp = (int)((t + 63) / 64 * 64);
  L->Epad = (int)((E + 63) / 64 * 64);
  L->Kc = (int)(2 * fs + l + (size_t)L->Epad);
  const size_t Kc = L->Kc;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up(o + bytes);
    return at;
  };
  const size_t rec = c->keep_preact ? 0 : 1;  // pre-activations recomputed here unless the forward kept them
  L->P = take(rec * t * fs * es);
  L->Q = take(rec * t * fs * es);
  L->dG = take(t * fs * es);
  L->dy = take(t * l * es);
  L->dAcat = take(t * Kc * es);
  L->dg = take(t * k * 4);
  L->dY = take(Tk * l * es);
  L->dH = take(Tk * f * es);
  L->Apre = take(rec * Tk * f * es);
  L->U = take(rec * Tk * f * es);
  L->dAU = take(Tk * 2 * f * es);
  L->dX = take(Tk * l * es);
  L->dh = take(t * d * 4);
  L->rstd = take(t * 4);
  L->gpart = take((size_t)kGammaSlices * d * 4);
  L->dWcat = take(std::max((size_t)kSplitOut * d * (fs + l), (size_t)kSplitCat * Kc * d) * 4);  // split-K partials
  L->total = o;
}

struct MxWeights {
  uint8_t *g8, *u8, *d8, *gs, *us, *ds;
};
// The block-scaled expert weights in the state: W_g, W_u, W_d elements (E4M3
// bytes, or E2M1 pairs for MXFP4), then their scale bytes.
MxWeights mx_weights(moe_ctx* ctx) {
  const size_t w = (size_t)ctx->cfg.E * ctx->cfg.f * ctx->cfg.l;
  const size_t wb = ctx->cfg.experts == MOE_EXPERTS_MXFP4 ? w / 2 : w;
  uint8_t* b = reinterpret_cast<uint8_t*>(ctx->state + ctx->sl.mx);
  return {b, b + wb, b + 2 * wb, b + 3 * wb, b + 3 * wb + w / 32, b + 3 * wb + 2 * (w / 32)};
}

hipError_t quantize_experts(moe_ctx* ctx, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  const MxWeights m = mx_weights(ctx);
  const bool w4 = c.experts == MOE_EXPERTS_MXFP4;
  const long long rows_gu = (long long)c.E * c.f, rows_d = (long long)c.E * c.l;
  hipError_t e = launch_mx_quant(ctx->w.W_g, rows_gu, c.l, c.l, m.g8, m.gs, s, w4);
  if (e == hipSuccess) e = launch_mx_quant(ctx->w.W_u, rows_gu, c.l, c.l, m.u8, m.us, s, w4);
  if (e == hipSuccess) e = launch_mx_quant(ctx->w.W_d, rows_d, c.f, c.f, m.d8, m.ds, s, w4);
  return e;
}

moe_status hip_ok(hipError_t e, const char* what) {
  return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t moe_state_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  moe_state_layout L;
  state_layout(cfg, &L);
  return L.total;
}

moe_status moe_state_layout_of(const moe_config* cfg, moe_state_layout* out) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "output is NULL");
  state_layout(cfg, out);
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_config(cfg) != MOE_OK || T < 0 || T > cfg->max_tokens) return 0;
  moe_ws_layout L;
  ws_layout(cfg, T, &L);
  return L.total;
}

moe_status moe_workspace_layout(const moe_config* cfg, int64_t T, moe_ws_layout* out) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "output is NULL");
  if (T < 0 || T > cfg->max_tokens) return fail(MOE_ERR_SHAPE, "T outside [0, max_tokens]");
  ws_layout(cfg, T, out);
  return MOE_OK;
}

moe_status moe_init(const moe_config* cfg, const moe_weights* w, void* state, void* stream, moe_ctx** out) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!w || !out) return fail(MOE_ERR_INVALID_ARG, "weights or output pointer is NULL");
  if (!w->gamma || !w->W_r || !w->W_dn || !w->W_g || !w->W_u || !w->W_d || !w->W_up)
    return fail(MOE_ERR_INVALID_ARG, "a required weight pointer is NULL");
  if (shared_hidden(cfg) > 0 && (!w->W_sg || !w->W_su || !w->W_sd))
    return fail(MOE_ERR_INVALID_ARG, "shared-expert weights are NULL while n_shared * f_s > 0");
  if (!state) return fail(MOE_ERR_INVALID_ARG, "state buffer is NULL");
  if (!aligned(state, kAlign)) return fail(MOE_ERR_INVALID_ARG, "state buffer must be 256-byte aligned");
  moe_ctx* c = new (std::nothrow) moe_ctx();
  if (!c) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  c->w = *w;
  c->state = static_cast<char*>(state);
  state_layout(cfg, &c->sl);
  c->D = dims_of(cfg);
  c->pending_tokens = 0;
  hipError_t e = launch_zero(state, c->sl.total, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && cfg->experts != MOE_EXPERTS_BF16) e = quantize_experts(c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete c;
    return fail(MOE_ERR_HIP, "clearing the state failed: %s", hipGetErrorString(e));
  }
  void* scratch_dev = nullptr;  // set up the no-alloc forward's scratch on this device
  if (scratch_of_current_device(&scratch_dev) != MOE_OK) {
    delete c;
    return MOE_ERR_HIP;
  }
  e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);  // default priority
  for (int i = 0; i < 4 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&c->fork_ev[i], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    moe_destroy(c);
    return fail(MOE_ERR_HIP, "creating the backward stream failed: %s", hipGetErrorString(e));
  }
  *out = c;
  return MOE_OK;
}

moe_status moe_route(moe_ctx* ctx, const void* x, const float* logits, int64_t T, moe_route_out* r, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status st = check_call(ctx, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!logits && !x) return fail(MOE_ERR_INVALID_ARG, "x and logits are both NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe_ws_layout L;
  ws_layout(&ctx->cfg, T, &L);
  char* w = static_cast<char*>(ws);
  RoutePtrs p = route_ptrs(ctx->cfg, T, L, w, r);
  const int t = (int)T;
  if (logits) {
    p.logits = const_cast<float*>(logits);
    // no RMSNorm launch to clear the super-chunk counts in: a fill launch
    MOE_RUN(MOE_K_SCAN, launch_zero(p.sbase, ((size_t)p.nsbase * 4 + 15) / 16 * 16, s));  // in the 256-byte padding
  } else {
    const Dims& D = ctx->D;
    void* h = w + L.h;
    MOE_RUN(MOE_K_RMSNORM, launch_rmsnorm(D, x, ctx->w.gamma, h, t, s, p.sbase, p.nsbase));
    MOE_RUN(MOE_K_GEMM_RZ, launch_gemm_rz(D, h, t, ctx->w.W_r, ctx->w.logit_offset, p.logits, s));
  }
  return route_tail(ctx, p, t, s);
}

moe_status moe_forward(moe_ctx* ctx, const void* x, int64_t T, void* out, moe_route_out* r, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_call(ctx, T, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "x or out is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& D = ctx->D;
  moe_ws_layout L;
  ws_layout(&ctx->cfg, T, &L);
  char* w = static_cast<char*>(ws);
  RoutePtrs p = route_ptrs(ctx->cfg, T, L, w, r);
  const int t = (int)T;
  void *h = w + L.h, *G = w + L.G, *z = w + L.z, *H = w + L.H, *Y = w + L.Y, *y_lat = w + L.y_lat;
  const bool keep = ctx->cfg.keep_preact != 0;
  MOE_RUN(MOE_K_RMSNORM, launch_rmsnorm(D, x, ctx->w.gamma, h, t, s, p.sbase, p.nsbase));
  MOE_RUN(MOE_K_GEMM_H, launch_gemm_h(D, h, t, ctx->w.W_r, ctx->w.logit_offset, ctx->w.W_sg, ctx->w.W_su,
                                      ctx->w.W_dn, p.logits, D.f_s > 0 ? G : nullptr, z, s,
                                      keep && D.f_s > 0 ? w + L.P : nullptr, keep && D.f_s > 0 ? w + L.Q : nullptr));
  const int32_t* n_mtiles = p.tile_offsets + D.E;
  if (ctx->cfg.experts != MOE_EXPERTS_BF16) {
    const bool w4 = ctx->cfg.experts == MOE_EXPERTS_MXFP4;
    // z -> MXFP8; the scatter copies each token's scale row to its grouped rows
    uint8_t *z8 = reinterpret_cast<uint8_t*>(w + L.z8), *zs = reinterpret_cast<uint8_t*>(w + L.zs);
    uint8_t *Xs = reinterpret_cast<uint8_t*>(w + L.Xs), *H8 = reinterpret_cast<uint8_t*>(w + L.H8);
    uint8_t* Hs = reinterpret_cast<uint8_t*>(w + L.Hs);
    const MxWeights m = mx_weights(ctx);
    MOE_RUN(MOE_K_MX_QUANT, launch_mx_quant(z, t, D.l, D.l, z8, zs, s));
    st = route_tail(ctx, p, t, s, zs, Xs);
    if (st != MOE_OK) return st;
    MOE_RUN(MOE_K_EXPERT_UP, launch_expert_up_mx(D, z8, Xs, p.perm_src, p.tile_info, n_mtiles, t, m.g8, m.gs, m.u8,
                                                 m.us, H, H8, Hs, s, w4));
    MOE_RUN(MOE_K_EXPERT_DOWN, launch_expert_down_mx(D, H8, Hs, p.tile_info, n_mtiles, t, m.d8, m.ds, Y, s, w4));
  } else {
    st = route_tail(ctx, p, t, s);
    if (st != MOE_OK) return st;
    // dispatch X[r] = z[perm_src[r]] happens inside expert_up's operand load
    // Many rows per expert (T k / E >= 512): 128-row tiles (better operand reuse); fewer: 64-row tiles
    // (128-row ones measured slower at 192 and 293 rows per expert, 8-14% faster at 768 and 3072).
    const bool tall = (long long)t * D.k >= 512LL * D.E;
    MOE_RUN(MOE_K_EXPERT_UP, launch_expert_up(D, z, p.perm_src, tall ? p.tile_info2 : p.tile_info,
                                              tall ? p.tile_offsets2 + D.E : n_mtiles, t, ctx->w.W_g, ctx->w.W_u, H,
                                              s, keep ? w + L.A : nullptr, keep ? w + L.U : nullptr, tall));
    MOE_RUN(MOE_K_EXPERT_DOWN,
            launch_expert_down(D, H, p.tile_info2, p.tile_offsets2 + D.E, t, ctx->w.W_d, Y, s));
  }
  MOE_RUN(MOE_K_COMBINE, launch_combine(D, Y, p.gates, p.inv, t, y_lat, s));
  MOE_RUN(MOE_K_GEMM_OUT, launch_gemm_out(D, G, y_lat, t, ctx->w.W_sd, ctx->w.W_up, out, s));
  return MOE_OK;
}

moe_status moe_forward_noalloc(moe_ctx* ctx, const void* x, int64_t T, void* out, moe_route_out* r, void* stream) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (T < 0 || T > ctx->cfg.max_tokens)
    return fail(MOE_ERR_SHAPE, "T=%lld outside [0, max_tokens=%lld]", (long long)T, (long long)ctx->cfg.max_tokens);
  const size_t need = moe_workspace_bytes(&ctx->cfg, T);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "T=%lld needs %zu bytes of workspace; the no-alloc forward has %zu (MOE_NOALLOC_SCRATCH_BYTES): "
                "call moe_forward with a workspace, or split the batch",
                (long long)T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return MOE_OK;
  void* ws = nullptr;
  moe_status st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  // nothing in the workspace has to start at zero: every piece a forward
  // reads is written earlier in the same forward
  return moe_forward(ctx, x, T, out, r, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status qb_update(moe_ctx* ctx, void* stream) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (ctx->cfg.qb_mode == MOE_QB_FROZEN) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& D = ctx->D;
  uint32_t* hist = reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.hist);
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(ctx->state + ctx->sl.count);
  double* q = reinterpret_cast<double*>(ctx->state + ctx->sl.q);
  float* bias = reinterpret_cast<float*>(ctx->state + ctx->sl.bias);
  if (ctx->cfg.balancer == MOE_BALANCE_SIGN) {
    uint32_t* load = reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.load);
    MOE_RUN(MOE_K_SIGN_BIAS, launch_sign_bias(D, load, cnt, ctx->cfg.sign_gamma, bias, s));
    ctx->pending_tokens = 0;
    return MOE_OK;
  }
  MOE_RUN(MOE_K_QB_UPDATE, launch_qb_update(D, hist, cnt, q, bias, s));
  ctx->pending_tokens = 0;
  return MOE_OK;
}

size_t moe_backward_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_config(cfg) != MOE_OK || T < 0 || T > cfg->max_tokens) return 0;
  BwdLayout L;
  bwd_layout(cfg, T, &L);
  return L.total;
}

moe_status moe_backward(moe_ctx* ctx, const void* x, const void* dout, int64_t T, const moe_route_out* r,
                        const void* fwd_ws, size_t fwd_ws_bytes, void* dx, const moe_grads* g, void* ws,
                        size_t ws_bytes, void* stream) {
  // a backward adds nothing to the training statistics
  moe_status st = check_call(ctx, T, const_cast<void*>(fwd_ws), fwd_ws_bytes, /*accumulates=*/false);
  if (st != MOE_OK || T == 0) return st;
  if (!x || !dout || !dx || !g) return fail(MOE_ERR_INVALID_ARG, "x, dout, dx or grads is NULL");
  if (ctx->cfg.experts != MOE_EXPERTS_BF16) return fail(MOE_ERR_STATE, "the backward pass needs bf16 experts");
  const moe_config& c = ctx->cfg;
  if (!g->gamma || !g->W_r || !g->W_dn || !g->W_g || !g->W_u || !g->W_d || !g->W_up ||
      (shared_hidden(&c) > 0 && (!g->W_sg || !g->W_su || !g->W_sd)))
    return fail(MOE_ERR_INVALID_ARG, "a required gradient pointer is NULL");
  BwdLayout B;
  bwd_layout(&c, T, &B);
  if (!ws || ws_bytes < B.total)
    return fail(MOE_ERR_WORKSPACE, "backward workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0,
                B.total);
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_WORKSPACE, "backward workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& D = ctx->D;
  const int t = (int)T, E = c.E, k = c.k, d = c.d, l = c.l, f = c.f, fs = shared_hidden(&c);
  const int es = c.dtype == MOE_BF16 ? 2 : 4;
  const int Tk = t * k, Tp = B.Tp, Kc = B.Kc, Epad = B.Epad;
  moe_ws_layout L;
  ws_layout(&c, T, &L);
  char* fw = static_cast<char*>(const_cast<void*>(fwd_ws));
  const RoutePtrs p = route_ptrs(ctx->cfg, T, L, fw, r);
  const void *h = fw + L.h, *G = fw + L.G, *z = fw + L.z, *H = fw + L.H, *Y = fw + L.Y, *y_lat = fw + L.y_lat;
  const int32_t* n_mtiles = p.tile_offsets + E;
  char* w = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(w + off); };
  void *P = at(B.P), *Q = at(B.Q);
  void *dG = at(B.dG), *dy = at(B.dy), *dAcat = at(B.dAcat), *dY = at(B.dY), *dH = at(B.dH), *Apre = at(B.Apre);
  void *U = at(B.U), *dAU = at(B.dAU), *dX = at(B.dX);
  float* dg = static_cast<float*>(at(B.dg));
  float* dh = static_cast<float*>(at(B.dh));
  float* dWcat = static_cast<float*>(at(B.dWcat));
  auto el = [&](const void* base, size_t elems) { return static_cast<const char*>(base) + elems * es; };
  auto elw = [&](void* base, size_t elems) { return static_cast<char*>(base) + elems * es; };
  const moe_weights& W = ctx->w;

  // With kept pre-activations the weight-gradient products run on an
  // internal stream, each forked off the caller's stream once its operands
  // are written there (the side stream's work stays in order: the dense ones
  // share the split-K partials), and joined back before returning; they then
  // overlap the chain of data gradients, much of which is bound by memory or
  // latency.  When the pre-activations are recomputed, those GEMMs already
  // fill the GPU beside the chain and everything stays on the caller's
  // stream (the overlap measured slower there).
  const bool kept = c.keep_preact != 0;  // pre-activations stored by the forward
  hipStream_t s2 = kept ? ctx->side : s;
  // Once forked, every return (an error included) leaves the caller's stream
  // waiting for the internal one, so no work of this call outlives it there.
  struct Join {
    hipStream_t s, s2;
    hipEvent_t ev;
    bool armed = false;
    ~Join() {
      if (armed) {
        (void)hipEventRecord(ev, s2);
        (void)hipStreamWaitEvent(s, ev, 0);
      }
    }
  } join{s, s2, ctx->join_ev};
  int nfork = 0;
  auto fork = [&]() -> moe_status {
    if (s2 == s) return MOE_OK;
    hipEvent_t ev = ctx->fork_ev[nfork++];
    hipError_t e = hipEventRecord(ev, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s2, ev, 0);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "forking the backward stream failed: %s", hipGetErrorString(e));
    join.armed = true;
    return MOE_OK;
  };
  const int u = Tp / 64;
  auto slices = [&](int want, int* step) {
    const int c = (u + want - 1) / want;  // 64-token stages per slice
    *step = 64 * c;
    return (u + c - 1) / c;               // every slice non-empty
  };
  int step_o, step_c;
  const int S_o = slices(kSplitOut, &step_o), S_c = slices(kSplitCat, &step_c);
  // [dW_sd | dW_up] = dout^T [G | y_lat]: forward values and dout only
  if ((st = fork()) != MOE_OK) return st;
  {
    hipStream_t s = s2;
    auto wgrad_out = [&]() -> hipError_t {
      WgradKmSpec wo{dout, d, G, fs, y_lat, l, fs, nullptr, step_o, t, nullptr, 0, d, fs + l, S_o, dWcat};
      hipError_t e = launch_wgrad_km(D, wo, s);
      SplitOut o{};
      o.by_rows = 0;
      auto addc = [&](int start, int len, float* out) {
        o.start[o.nseg] = start;
        o.len[o.nseg] = len;
        o.ld[o.nseg] = len;
        o.out[o.nseg] = out;
        ++o.nseg;
      };
      if (fs > 0) addc(0, fs, g->W_sd);
      addc(fs, l, g->W_up);
      if (e == hipSuccess) e = launch_reduce_split(dWcat, S_o, d, fs + l, o, s);
      return e;
    };
    MOE_RUN(MOE_K_BWD_WGRAD, wgrad_out());
  }
  // Data-gradient products read the weights as stored (K-major B operands).
  // output projections: [dG | dy_lat] = dout [W_sd | W_up]
  {
    DgradSegSpec sg[2] = {};
    int n = 0;
    if (fs > 0) sg[n++] = {{{W.W_sd, fs, d, d}}, fs, 1, dG, fs};
    sg[n++] = {{{W.W_up, l, d, d}}, l, 1, dy, l};
    MOE_RUN(MOE_K_BWD_GEMM, launch_dgrad_dense(D, 4, dout, d * es, t, sg, n, 1, s));
  }
  if (kept) {
    P = fw + L.P;
    Q = fw + L.Q;
    Apre = fw + L.A;
    U = fw + L.U;
  }
  if (fs > 0) {  // shared GLU: P, Q (recomputed unless kept); dP, dQ into the first 2 f_s columns of dAcat
    if (!kept) {
      DenseSegSpec sg[2] = {{W.W_sg, fs, 1, P, fs}, {W.W_su, fs, 1, Q, fs}};
      MOE_RUN(MOE_K_BWD_GEMM, launch_dense_nt(D, 3, h, d * es, t, d * es, sg, 2, d * es, s));
    }
    MOE_RUN(MOE_K_BWD_ELTWISE, launch_glu_bwd(D, P, Q, dG, t, fs, dAcat, elw(dAcat, fs), Kc, s));
  }
  // expert pre-activations A = X W_g^T, U = X W_u^T (recomputed unless kept),
  // before the next fork so that they do not share the GPU with its products
  const size_t wfl = (size_t)f * l * es;
  if (!kept) {
    MOE_RUN(MOE_K_BWD_EXPERT, launch_expert_nt(D, z, l * es, p.perm_src, W.W_g, wfl, l * es, f, l * es, p.tile_info,
                                               n_mtiles, t, Apre, f, s));
    MOE_RUN(MOE_K_BWD_EXPERT, launch_expert_nt(D, z, l * es, p.perm_src, W.W_u, wfl, l * es, f, l * es, p.tile_info,
                                               n_mtiles, t, U, f, s));
  }
  // combine transpose: dY rows and gate gradients
  MOE_RUN(MOE_K_BWD_ELTWISE, launch_combine_bwd(D, dy, Y, p.gates, p.inv, t, dY, dg, s));
  // dW_d[e] = dY_e^T H_e (K = the expert's rows of the dispatch order)
  if ((st = fork()) != MOE_OK) return st;
  {
    hipStream_t s = s2;
    const WgradKmSpec wd{dY, l, nullptr, 0, H, f, 0, p.offsets, 0, Tk, nullptr, 0, l, f, E, g->W_d};
    MOE_RUN(MOE_K_BWD_WGRAD, launch_wgrad_km(D, wd, s));
  }
  // experts: dH = dY W_d; GLU derivative; dX = [dA|dU] [W_g; W_u]
  {
    const KPiece wd[1] = {{W.W_d, f, l, l}};  // W_d[e] [l, f]: K = l
    MOE_RUN(MOE_K_BWD_EXPERT,
            launch_dgrad_expert(D, 8, dY, l * es, wd, 1, wfl, f, p.tile_info, n_mtiles, t, dH, f, s));
  }
  MOE_RUN(MOE_K_BWD_ELTWISE, launch_glu_bwd(D, Apre, U, dH, Tk, f, dAU, elw(dAU, f), 2 * f, s));
  // dW_g[e] = dA_e^T X_e and dW_u[e] = dU_e^T X_e, X_e's rows gathered from z
  if ((st = fork()) != MOE_OK) return st;
  {
    hipStream_t s = s2;
    const WgradKmSpec wg{dAU, 2 * f, nullptr, 0, z, l, 0, p.offsets, 0, Tk, p.perm_src, Tk, f, l, E, g->W_g};
    MOE_RUN(MOE_K_BWD_WGRAD, launch_wgrad_km(D, wg, s));
    WgradKmSpec wu = wg;
    wu.A = el(dAU, f);
    wu.out = g->W_u;
    MOE_RUN(MOE_K_BWD_WGRAD, launch_wgrad_km(D, wu, s));
  }
  {
    const KPiece wgu[2] = {{W.W_g, l, f, f}, {W.W_u, l, f, f}};  // [W_g[e]; W_u[e]] [2f, l]: K = 2f
    MOE_RUN(MOE_K_BWD_EXPERT,
            launch_dgrad_expert(D, 9, dAU, 2 * f * es, wgu, 2, wfl, l, p.tile_info, n_mtiles, t, dX, l, s));
  }
  // dispatch transpose and router: dz and dl into their columns of dAcat
  MOE_RUN(MOE_K_BWD_ELTWISE, launch_dispatch_bwd(D, dX, p.inv, t, elw(dAcat, 2 * fs), Kc, s));
  MOE_RUN(MOE_K_BWD_ELTWISE, launch_gates_bwd(D, p.logits, p.idx, dg, t, Epad, elw(dAcat, 2 * fs + l), Kc, s));
  // [dW_sg; dW_su; dW_dn; dW_r] = dA_cat^T h, K = tokens in slices, partials summed into the outputs
  if ((st = fork()) != MOE_OK) return st;
  {
    hipStream_t s = s2;
    auto wgrad_cat = [&]() -> hipError_t {
      WgradKmSpec wc{dAcat, Kc, nullptr, 0, h, d, 0, nullptr, step_c, t, nullptr, 0, Kc, d, S_c, dWcat};
      hipError_t e = launch_wgrad_km(D, wc, s);
      SplitOut c{};
      c.by_rows = 1;
      auto add = [&](int start, int len, float* out) {
        c.start[c.nseg] = start;
        c.len[c.nseg] = len;
        c.ld[c.nseg] = d;
        c.out[c.nseg] = out;
        ++c.nseg;
      };
      if (fs > 0) {
        add(0, fs, g->W_sg);
        add(fs, fs, g->W_su);
      }
      add(2 * fs, l, g->W_dn);
      add(2 * fs + l, E, g->W_r);
      if (e == hipSuccess) e = launch_reduce_split(dWcat, S_c, Kc, d, c, s);
      return e;
    };
    MOE_RUN(MOE_K_BWD_WGRAD, wgrad_cat());
  }
  // dh = [dP | dQ | dz | dl] [W_sg; W_su; W_dn; W_r], then RMSNorm
  {
    DgradSegSpec sg = {};
    int np = 0;
    if (fs > 0) {
      sg.piece[np++] = {W.W_sg, d, fs, fs};
      sg.piece[np++] = {W.W_su, d, fs, fs};
    }
    sg.piece[np++] = {W.W_dn, d, l, l};
    sg.piece[np++] = {W.W_r, d, Epad, E};  // pad rows of W_r count as zero
    sg.N = d;
    sg.kind = 0;
    sg.out = dh;
    sg.ldo = d;
    MOE_RUN(MOE_K_BWD_GEMM, launch_dgrad_dense(D, 5, dAcat, Kc * es, t, &sg, 1, np, s));
  }
  MOE_RUN(MOE_K_BWD_ELTWISE, launch_rmsnorm_bwd(D, x, W.gamma, dh, t, dx, static_cast<float*>(at(B.rstd)),
                                                static_cast<float*>(at(B.gpart)), kGammaSlices, g->gamma, s));
  // join: the caller's stream waits for the weight gradients
  if (join.armed) {
    join.armed = false;
    hipError_t e = hipEventRecord(ctx->join_ev, s2);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ctx->join_ev, 0);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "joining the backward stream failed: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

moe_status moe_requantize_experts(moe_ctx* ctx, void* stream) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (ctx->cfg.experts == MOE_EXPERTS_BF16) return MOE_OK;
  return hip_ok(quantize_experts(ctx, static_cast<hipStream_t>(stream)), "expert quantisation");
}

moe_status moe_get_bias(moe_ctx* ctx, float* dst, void* stream) {
  if (!ctx || !dst) return fail(MOE_ERR_INVALID_ARG, "context or destination is NULL");
  hipError_t e = hipMemcpyAsync(dst, ctx->state + ctx->sl.bias, (size_t)ctx->cfg.E * 4, hipMemcpyDefault,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "bias copy failed: %s", hipGetErrorString(e));
}

moe_status moe_set_bias(moe_ctx* ctx, const float* src, void* stream) {
  if (!ctx || !src) return fail(MOE_ERR_INVALID_ARG, "context or source is NULL");
  hipError_t e = hipMemcpyAsync(ctx->state + ctx->sl.bias, src, (size_t)ctx->cfg.E * 4, hipMemcpyDefault,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : fail(MOE_ERR_HIP, "bias copy failed: %s", hipGetErrorString(e));
}

moe_status moe_fast_score_error(float* err, void* stream) {
  if (!err) return fail(MOE_ERR_INVALID_ARG, "destination is NULL");
  return hip_ok(launch_fast_score_error(err, static_cast<hipStream_t>(stream)), "fast score check");
}

moe_status moe_set_qb_mode(moe_ctx* ctx, moe_qb_mode mode) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (mode != MOE_QB_TRAIN && mode != MOE_QB_FROZEN) return fail(MOE_ERR_INVALID_ARG, "unknown qb_mode");
  ctx->cfg.qb_mode = mode;
  return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : ctx->fork_ev)
    if (e) (void)hipEventDestroy(e);
  if (ctx->join_ev) (void)hipEventDestroy(ctx->join_ev);
  if (ctx->side) (void)hipStreamDestroy(ctx->side);
  delete ctx;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_STATE: return "MOE_ERR_STATE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

const char* moe_kernel_name(int id) {
  static const char* names[MOE_NUM_KERNELS] = {"rmsnorm",     "gemm_h",  "topk",     "hist",
                                                "scan",        "scatter", "expert_up", "expert_down",
                                                "combine",     "gemm_out", "qb_update", "qb_bias", "gemm_rz",
                                                "sign_bias",   "bwd_gemm", "bwd_expert", "bwd_wgrad",
                                                "bwd_eltwise", "bwd_transpose", "mx_quant"};
  return (id >= 0 && id < MOE_NUM_KERNELS) ? names[id] : "unknown";
}

moe_status moe_profile_begin(moe_ctx* ctx, int max_launches, uint32_t mask) {
  if (!ctx || max_launches < 1) return fail(MOE_ERR_INVALID_ARG, "bad profiling arguments");
  if ((int)ctx->ev.size() < 2 * max_launches) {
    while ((int)ctx->ev.size() < 2 * max_launches) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreate failed");
      ctx->ev.push_back(e);
    }
  }
  ctx->ev_kernel.assign(max_launches, -1);
  ctx->prof_mask = mask;
  ctx->prof_max = max_launches;
  ctx->prof_n = 0;
  ctx->prof = true;
  return MOE_OK;
}

moe_status moe_profile_end(moe_ctx* ctx, double* ms, int64_t* launches, int n) {
  if (!ctx || !ms || !launches || n < 1) return fail(MOE_ERR_INVALID_ARG, "bad profiling arguments");
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  moe_status st = MOE_OK;
  for (int i = 0; i < ctx->prof_n; ++i) {
    if (hipEventSynchronize(ctx->ev[2 * i + 1]) != hipSuccess) {
      st = fail(MOE_ERR_HIP, "hipEventSynchronize failed");
      break;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, ctx->ev[2 * i], ctx->ev[2 * i + 1]) != hipSuccess) {
      st = fail(MOE_ERR_HIP, "hipEventElapsedTime failed");
      break;
    }
    const int k = ctx->ev_kernel[i];
    if (k >= 0 && k < n) {
      ms[k] += t;
      launches[k] += 1;
    }
  }
  ctx->prof = false;
  ctx->prof_n = 0;
  return st;
}

}  // extern "C"
