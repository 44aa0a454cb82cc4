// C ABI of the LatentMoE layer (include/moe.h): argument checks, workspace
// and state layouts, the launch sequence of a forward / routing pass / QB
// update, and optional per-kernel event timing.  Host code only; all device
// memory belongs to the caller.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <vector>

#include "kernels.h"

using namespace moe;

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

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "unknown dtype %d", (int)c->dtype);
  if (c->qb_mode != MOE_QB_TRAIN && c->qb_mode != MOE_QB_FROZEN)
    return fail(MOE_ERR_INVALID_ARG, "unknown qb_mode %d", (int)c->qb_mode);
  if (c->balancer != MOE_BALANCE_QB && c->balancer != MOE_BALANCE_SIGN)
    return fail(MOE_ERR_INVALID_ARG, "unknown balancer %d", (int)c->balancer);
  if (c->balancer == MOE_BALANCE_SIGN && !(c->sign_gamma > 0.f && std::isfinite(c->sign_gamma)))
    return fail(MOE_ERR_INVALID_ARG, "sign_gamma must be finite and > 0");
  auto m64 = [](int32_t v) { return v > 0 && v % 64 == 0; };
  if (!m64(c->d) || !m64(c->l) || !m64(c->f))
    return fail(MOE_ERR_SHAPE, "d, l, f must be positive multiples of 64 (d=%d l=%d f=%d)", c->d, c->l, c->f);
  if (c->f_s < 0 || c->f_s % 64 != 0) return fail(MOE_ERR_SHAPE, "f_s must be 0 or a multiple of 64 (f_s=%d)", c->f_s);
  if (c->d > (1 << 20) || c->l > (1 << 20) || c->f > (1 << 20) || c->f_s > (1 << 20))
    return fail(MOE_ERR_SHAPE, "a width exceeds 2^20");
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
  D.f_s = c->f_s;
  D.B = c->qb_bins;
  D.bf16 = c->dtype == MOE_BF16;
  D.eps = c->rms_eps;
  D.routed_scale = c->routed_scale;
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
  L->hist_slices = kHistSlices;
  o = up(o + (size_t)kHistSlices * c->E * c->qb_bins * 4);
  L->load = o;
  o = up(o + (size_t)c->E * 4);
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
  L->cbase = take(nchunks * E * 4);
  L->sbase = take(nsuper * E * 4);
  L->counts = take(E * 4);
  L->offsets = take((E + 1) * 4);
  L->tile_offsets = take((E + 1) * 4);
  L->perm_src = take(t * k * 4);
  L->inv = take(t * k * 4);
  L->tile_info = take(T > 0 ? (size_t)expert_max_mtiles((int)T, c->k, c->E) * 8 : 0);
  L->G = take(t * c->f_s * es);
  L->z = take(t * c->l * es);
  L->X = take(0);  // no dispatch buffer: expert_up gathers z rows itself
  L->H = take(t * k * c->f * es);
  L->Y = take(t * k * c->l * es);
  L->y_lat = take(t * c->l * es);
  L->total = o;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

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
  int32_t *idx, *cbase, *sbase, *counts, *offsets, *tile_offsets, *perm_src, *inv;
  uint32_t* bitmap;
  int2* tile_info;
  float* gates;
};

RoutePtrs route_ptrs(const moe_ws_layout& L, char* ws, const moe_route_out* r) {
  RoutePtrs p;
  p.logits = (r && r->logits) ? r->logits : reinterpret_cast<float*>(ws + L.logits);
  p.idx = (r && r->topk_idx) ? r->topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  p.gates = (r && r->gates) ? r->gates : reinterpret_cast<float*>(ws + L.gates);
  p.counts = (r && r->counts) ? r->counts : reinterpret_cast<int32_t*>(ws + L.counts);
  p.offsets = (r && r->offsets) ? r->offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  p.perm_src = (r && r->perm_src) ? r->perm_src : reinterpret_cast<int32_t*>(ws + L.perm_src);
  p.inv = (r && r->inv) ? r->inv : reinterpret_cast<int32_t*>(ws + L.inv);
  p.bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  p.cbase = reinterpret_cast<int32_t*>(ws + L.cbase);
  p.sbase = reinterpret_cast<int32_t*>(ws + L.sbase);
  p.tile_offsets = reinterpret_cast<int32_t*>(ws + L.tile_offsets);
  p.tile_info = reinterpret_cast<int2*>(ws + L.tile_info);
  return p;
}

moe_status check_call(moe_ctx* ctx, int64_t T, void* ws, size_t ws_bytes) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (T < 0 || T > ctx->cfg.max_tokens)
    return fail(MOE_ERR_SHAPE, "T=%lld outside [0, max_tokens=%lld]", (long long)T, (long long)ctx->cfg.max_tokens);
  if (T == 0) return MOE_OK;
  const size_t need = moe_workspace_bytes(&ctx->cfg, T);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ctx->cfg.qb_mode == MOE_QB_TRAIN && ctx->pending_tokens + (uint64_t)T >= (uint64_t(1) << 32))
    return fail(MOE_ERR_STATE, "more than 2^32-1 tokens accumulated without qb_update");
  return MOE_OK;
}

// Steps after the logits: scores, QB histogram, top-k + gates + selection
// masks, two-level prefix sums with offsets, stable rows (perm_src, inv).
moe_status route_tail(moe_ctx* ctx, const RoutePtrs& p, int T, hipStream_t s) {
  const Dims& D = ctx->D;
  const float* bias = reinterpret_cast<const float*>(ctx->state + ctx->sl.bias);
  const bool train = ctx->cfg.qb_mode == MOE_QB_TRAIN;
  const bool sign = ctx->cfg.balancer == MOE_BALANCE_SIGN;
  // training statistics: the score histogram (QB) or the per-expert loads (sign rule)
  uint32_t* hist = train && !sign ? reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.hist) : nullptr;
  uint32_t* load = train && sign ? reinterpret_cast<uint32_t*>(ctx->state + ctx->sl.load) : nullptr;
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(ctx->state + ctx->sl.count);
  MOE_RUN(MOE_K_TOPK, launch_topk(D, p.logits, bias, T, p.idx, p.gates, p.bitmap, hist, cnt, s));
  if (train) ctx->pending_tokens += (uint64_t)T;
  MOE_RUN(MOE_K_SCAN, launch_scan(D, p.bitmap, T, p.cbase, p.sbase, p.counts, p.offsets, p.tile_offsets,
                                  p.tile_info, load, train && sign ? cnt : nullptr, s));
  MOE_RUN(MOE_K_SCATTER, launch_scatter(D, p.idx, p.bitmap, p.cbase, p.sbase, T, p.perm_src, p.inv, s));
  return MOE_OK;
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
  if (cfg->f_s > 0 && (!w->W_sg || !w->W_su || !w->W_sd))
    return fail(MOE_ERR_INVALID_ARG, "shared-expert weights are NULL while f_s > 0");
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
  if (e != hipSuccess) {
    delete c;
    return fail(MOE_ERR_HIP, "clearing the state failed: %s", hipGetErrorString(e));
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
  RoutePtrs p = route_ptrs(L, w, r);
  const int t = (int)T;
  if (logits) {
    p.logits = const_cast<float*>(logits);
  } else {
    const Dims& D = ctx->D;
    void* h = w + L.h;
    MOE_RUN(MOE_K_RMSNORM, launch_rmsnorm(D, x, ctx->w.gamma, h, t, s));
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
  RoutePtrs p = route_ptrs(L, w, r);
  const int t = (int)T;
  void *h = w + L.h, *G = w + L.G, *z = w + L.z, *H = w + L.H, *Y = w + L.Y, *y_lat = w + L.y_lat;
  MOE_RUN(MOE_K_RMSNORM, launch_rmsnorm(D, x, ctx->w.gamma, h, t, s));
  MOE_RUN(MOE_K_GEMM_H, launch_gemm_h(D, h, t, ctx->w.W_r, ctx->w.logit_offset, ctx->w.W_sg, ctx->w.W_su,
                                      ctx->w.W_dn, p.logits, D.f_s > 0 ? G : nullptr, z, s));
  st = route_tail(ctx, p, t, s);
  if (st != MOE_OK) return st;
  const int32_t* n_mtiles = p.tile_offsets + D.E;
  // dispatch X[r] = z[perm_src[r]] happens inside expert_up's operand load
  MOE_RUN(MOE_K_EXPERT_UP,
          launch_expert_up(D, z, p.perm_src, p.tile_info, n_mtiles, t, ctx->w.W_g, ctx->w.W_u, H, s));
  MOE_RUN(MOE_K_EXPERT_DOWN, launch_expert_down(D, H, p.tile_info, n_mtiles, t, ctx->w.W_d, Y, s));
  MOE_RUN(MOE_K_COMBINE, launch_combine(D, Y, p.gates, p.inv, t, y_lat, s));
  MOE_RUN(MOE_K_GEMM_OUT, launch_gemm_out(D, G, y_lat, t, ctx->w.W_sd, ctx->w.W_up, out, s));
  return MOE_OK;
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
  MOE_RUN(MOE_K_QB_QUANTILE, launch_qb_quantile(D, hist, cnt, q, s));
  MOE_RUN(MOE_K_QB_BIAS, launch_qb_bias(D, q, cnt, bias, s));
  ctx->pending_tokens = 0;
  return MOE_OK;
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

moe_status moe_set_qb_mode(moe_ctx* ctx, moe_qb_mode mode) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "context is NULL");
  if (mode != MOE_QB_TRAIN && mode != MOE_QB_FROZEN) return fail(MOE_ERR_INVALID_ARG, "unknown qb_mode");
  ctx->cfg.qb_mode = mode;
  return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->ev) (void)hipEventDestroy(e);
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
                                                "combine",     "gemm_out", "qb_quantile", "qb_bias", "gemm_rz",
                                                "sign_bias"};
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
