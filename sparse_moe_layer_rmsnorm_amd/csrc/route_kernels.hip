// Memory- and latency-bound kernels of the LatentMoE layer on gfx950:
// RMSNorm, router scores + biased top-k + gates, the QB score histogram,
// the count / scan / scatter token permutation, the gate-weighted combine,
// and the QB bias update.
//
// Sources (page title + place): "Kimi K3 MoE lightweight replica demo"
// article (architecture paragraph: width separation and the shared/routed
// dual path; Tab 2 Fig. 2(b): histogram quantile; Tab 8-10: the bias
// reroutes only, gates renormalised, update delayed, mean-centred, frozen at
// inference); "Pretraining a Mini Kimi K3" review, capsule 16 (bias rule,
// dead-expert lesson) and capsule 25 (dispatch buffer must never fall back
// silently); "K3 tops open source" blog, idle-experts section (hot experts
// raise their threshold).
#include "device_common.h"
#include "kernels.h"
#include "moe.h"

namespace moe {

static_assert(kFastScoreErr == MOE_FAST_SCORE_ERR, "the documented fast-score bound is the kernels' bound");

// ------------------------------------------------------------- RMSNorm ----
// One wavefront per token row; h = (x * rstd) * gamma, rstd = 1/sqrt(mean(x^2)
// + eps), fp32 arithmetic, stored in the activation dtype.  Rows of up to
// 64*CPL 16-byte chunks are read once into registers (all loads in flight
// together); longer rows take the two-pass loop (CPL = 0).
template <bool BF16>
MOE_DEV float chunk_sumsq(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      const float a = bf16_bits_to_f32(w[i] & 0xFFFFu), b = bf16_bits_to_f32(w[i] >> 16);
      ss += a * a + b * b;
    } else {
      const float a = __uint_as_float(w[i]);
      ss += a * a;
    }
  }
  return ss;
}

// gamma of one 16-byte chunk of the row (8 bf16 or 4 fp32 elements)
template <bool BF16>
struct ChunkGamma {
  float4 g0, g1;
};
template <bool BF16>
MOE_DEV ChunkGamma<BF16> chunk_gamma(const float* g) {
  ChunkGamma<BF16> r;
  r.g0 = *reinterpret_cast<const float4*>(g);
  r.g1 = BF16 ? *reinterpret_cast<const float4*>(g + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  return r;
}

template <bool BF16>
MOE_DEV uint4 chunk_scale(const uint4& v, float rstd, const ChunkGamma<BF16>& cg) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  if (BF16) {
    const float4 g0 = cg.g0, g1 = cg.g1;
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(bf16_bits_to_f32(w[i] & 0xFFFFu) * rstd * gg[2 * i],
                         bf16_bits_to_f32(w[i] >> 16) * rstd * gg[2 * i + 1]);
  } else {
    const float4 g0 = cg.g0;
    const float gg[4] = {g0.x, g0.y, g0.z, g0.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(w[i]) * rstd * gg[i]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <bool BF16, int CPL>
__global__ __launch_bounds__(256) void k_rmsnorm(const void* __restrict__ x, const float* __restrict__ gamma,
                                                 void* __restrict__ h, int T, int d, float eps,
                                                 int32_t* __restrict__ zero, int nzero) {
  // the top-k launch of the same pass accumulates into `zero` (per super-chunk
  // selection counts): cleared here, the pass's first launch
  for (int i = blockIdx.x * 256 + threadIdx.x; i < nzero; i += gridDim.x * 256) zero[i] = 0;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nch = d / EPC;
  const size_t rbytes = (size_t)d * (BF16 ? 2 : 4);
  const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + (size_t)row * rbytes);
  uint4* hr = reinterpret_cast<uint4*>(static_cast<char*>(h) + (size_t)row * rbytes);
  float ss = 0.f;
  if constexpr (CPL > 0) {
    uint4 v[CPL];
    ChunkGamma<BF16> g[CPL];  // gamma read with the row, not after its reduction
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      v[i] = c < nch ? xr[c] : make_uint4(0, 0, 0, 0);
      if (c < nch) g[i] = chunk_gamma<BF16>(gamma + c * EPC);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) ss += chunk_sumsq<BF16>(v[i]);
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) hr[c] = chunk_scale<BF16>(v[i], rstd, g[i]);
    }
  } else {
    for (int c = lane; c < nch; c += 64) ss += chunk_sumsq<BF16>(xr[c]);
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < nch; c += 64)
      hr[c] = chunk_scale<BF16>(xr[c], rstd, chunk_gamma<BF16>(gamma + c * EPC));
  }
}

template <bool BF16>
static void rmsnorm_dispatch(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s,
                             int32_t* zero, int nzero) {
  const int per_lane = (D.d / (BF16 ? 8 : 4) + 63) / 64;
  dim3 grid((T + 3) / 4), block(256);
#define MOE_RMS(C) \
  hipLaunchKernelGGL((k_rmsnorm<BF16, C>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps, zero, nzero)
  if (per_lane <= 1) MOE_RMS(1);
  else if (per_lane <= 2) MOE_RMS(2);
  else if (per_lane <= 4) MOE_RMS(4);
  else if (per_lane <= 8) MOE_RMS(8);
  else MOE_RMS(0);
#undef MOE_RMS
}

hipError_t launch_rmsnorm(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s,
                          int32_t* zero, int nzero) {
  if (T <= 0) return hipSuccess;
  if (D.bf16)
    rmsnorm_dispatch<true>(D, x, gamma, h, T, s, zero, nzero);
  else
    rmsnorm_dispatch<false>(D, x, gamma, h, T, s, zero, nzero);
  return hipGetLastError();
}

// -------------------------------------------------- scores + top-k ----
// Tokens are ranked in chunks of kChunk = 32, one chunk per block.
// The selection is the candidate filter below (topk_filter_tokens, or
// topk_group_tokens with 16 or 32 lanes per token); tokens it cannot settle
// take the k-round path here: lane i holds experts i, i+64, ...; each of the
// k rounds takes the wave-wide maximum (DPP, no LDS) of the order key of
// v = s + b; among equal keys the lowest expert index wins (first the lowest
// column c of any lane holding the key, then the lowest such lane, by
// ballots).  Gates are the chosen unbiased scores over their fp32 sum in
// slot order.  The chunk's selections leave as one 32-bit token mask per
// expert: bitmap[chunk][e] bit t%32 is set iff token t picked e.
template <int CPL, int NT>
MOE_DEV void topk_tokens(const float* __restrict__ logits, const float* sb, const int (&t)[NT], int E, int k,
                         float scale, int32_t* __restrict__ idx, float* __restrict__ gates, uint32_t* mask) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  float s[NT][CPL];
  uint32_t key[NT][CPL];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float* lr = logits + (size_t)t[n] * E;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      s[n][c] = e < E ? lr[e] : 0.f;
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      if (e < E) {
        s[n][c] = router_sigmoid(s[n][c]);
        key[n][c] = float_order_key(s[n][c] + sb[e]);  // > 0 for any finite v
      } else {
        s[n][c] = 0.f;
        key[n][c] = 0u;
      }
    }
  float S[NT], my_s[NT];
  int my_e[NT];
  for (int j = 0; j < k; ++j) {
    uint32_t best[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      best[n] = key[n][0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) best[n] = max(best[n], key[n][c]);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) best[n] = wave_max_u32(best[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      int sel_c = 0;
      unsigned long long sel = 0;
#pragma unroll
      for (int c = CPL - 1; c >= 0; --c) {
        const unsigned long long m = __ballot(key[n][c] == best[n]);
        if (m) {
          sel = m;
          sel_c = c;
        }
      }
      const int owner = (int)__builtin_ctzll(sel);
      float sv = s[n][0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) sv = (c == sel_c) ? s[n][c] : sv;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (c == sel_c && lane == owner) key[n][c] = 0u;
      const float se = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), owner));
      S[n] = (j == 0) ? se : S[n] + se;
      if (lane == j) {
        my_s[n] = se;
        my_e[n] = sel_c * 64 + owner;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
    if (lane < k) {
      const float g = (my_s[n] / S[n]) * scale;
      idx[(size_t)t[n] * k + lane] = my_e[n];
      gates[(size_t)t[n] * k + lane] = g;
      atomicOr(&mask[my_e[n]], 1u << (t[n] & 31));
    }
}

// Candidate filter in front of the exact ranking (same result as
// topk_tokens, bit for bit).  With fast scores v' = fast_sigmoid(l) + b, let
// tau be the k-th largest of the maxima of v' over G groups of 64/G lanes
// (G >= 2k, fewer groups make tau cheaper to find): at least k experts have
// v' >= tau, so the exact k-th largest v is >= tau - eps and every expert of
// the exact top-k has v' >= tau - 2 eps (eps bounds |v' - v|).
// The experts with v' >= tau - margin (margin >= 2 eps) are compacted into
// the wavefront's LDS, one per lane, and only they get the exact score; each
// candidate's slot is its rank among them by (exact key, lowest expert).
// A token with more than 64 candidates (many equal scores) or fewer than k
// (impossible while the error bound holds) takes the k-round path instead.
struct TopkScratch {            // one token's exchange area in LDS
  int32_t m[64];                // lane maxima of the fast keys; then the chosen scores in slot order
  float cl[64];                 // candidates: logit
  int32_t ce[64];               // candidates: expert
  unsigned long long r[64];     // candidates: (exact key << 32) | ~expert
};

template <int CPL, int NT>
MOE_DEV void topk_filter_tokens(const float* __restrict__ logits, const float* sb, const int (&t)[NT], int E,
                                int k, float scale, int32_t* __restrict__ idx, float* __restrict__ gates,
                                uint32_t* mask, TopkScratch* ts, bool (&fallback)[NT]) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  float l[NT][CPL];
  int32_t q[NT][CPL];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float* lr = logits + (size_t)t[n] * E;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      l[n][c] = e < E ? lr[e] : 0.f;
    }
  }
  int32_t mx[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) mx[n] = INT32_MIN;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    const float bc = e < E ? sb[e] : 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      q[n][c] = e < E ? float_skey(fast_sigmoid(l[n][c]) + bc) : INT32_MIN;
      mx[n] = max(mx[n], q[n][c]);
    }
  }
  // group maxima: lanes 4g .. 4g+3 (G = 16), 2g, 2g+1 (G = 32) or each lane
  const int G = k <= 8 ? 16 : k <= 16 ? 32 : 64;
  const int gs = 64 / G;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (gs >= 2) mx[n] = max(mx[n], __builtin_amdgcn_update_dpp(mx[n], mx[n], 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    if (gs >= 4) mx[n] = max(mx[n], __builtin_amdgcn_update_dpp(mx[n], mx[n], 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    if ((lane & (gs - 1)) == 0) ts[n].m[lane / gs] = mx[n];
  }
  wave_lds_sync();
  // tau: the smallest group maximum with fewer than k larger ones
  int32_t thr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int cnt = 0;
    for (int i = 0; i < G; i += 4) {
      const int4 w = *reinterpret_cast<const int4*>(&ts[n].m[i]);
      cnt += (w.x > mx[n]) + (w.y > mx[n]) + (w.z > mx[n]) + (w.w > mx[n]);
    }
    const int32_t tau = wave_min_i32(cnt < k ? mx[n] : INT32_MAX);
    const float vt = skey_float(tau);
    // margin: 2^-12 + 2^-16 |tau| >> 2 kFastScoreErr plus the roundings of v' and v
    thr[n] = __builtin_isfinite(vt) ? float_skey(vt - (0x1p-12f + fabsf(vt) * 0x1p-16f)) : INT32_MIN + 1;
  }
  int C[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int base = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const bool p = q[n][c] >= thr[n];
      const unsigned long long bm = __ballot(p);
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      if (p && pos < 64) {
        ts[n].cl[pos] = l[n][c];
        ts[n].ce[pos] = lane + 64 * c;
      }
      base += __popcll(bm);
    }
    C[n] = base;
    fallback[n] = base < k || base > 64;
  }
  wave_lds_sync();
  float s[NT];
  int e[NT];
  unsigned long long R[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    s[n] = 0.f;
    e[n] = 0;
    R[n] = 0ull;
    if (!fallback[n] && lane < C[n]) {
      e[n] = ts[n].ce[lane];
      s[n] = router_sigmoid(ts[n].cl[lane]);
      R[n] = ((unsigned long long)float_order_key(s[n] + sb[e[n]]) << 32) | (uint32_t)~e[n];
    }
    ts[n].r[lane] = R[n];  // lanes past the candidates write 0, below every real key
  }
  wave_lds_sync();
  int rank[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    rank[n] = 0;
    if (!fallback[n])
      for (int i = 0; i < C[n]; i += 2) {
        const ulonglong2 w = *reinterpret_cast<const ulonglong2*>(&ts[n].r[i]);
        rank[n] += (w.x > R[n]) + (w.y > R[n]);
      }
  }
  wave_lds_sync();
#pragma unroll
  for (int n = 0; n < NT; ++n)
    if (!fallback[n] && lane < C[n] && rank[n] < k) ts[n].m[rank[n]] = __float_as_int(s[n]);
  wave_lds_sync();
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (fallback[n]) continue;
    float S = __int_as_float(ts[n].m[0]);  // the gates' denominator: fp32 sum in slot order
    for (int j = 1; j < k; ++j) S = S + __int_as_float(ts[n].m[j]);
    if (lane < C[n] && rank[n] < k) {
      const size_t o = (size_t)t[n] * k + rank[n];
      idx[o] = e[n];
      gates[o] = (s[n] / S) * scale;
      atomicOr(&mask[e[n]], 1u << (t[n] & 31));
    }
  }
  wave_lds_sync();
}

#ifndef MOE_TOPK_NT
#define MOE_TOPK_NT 2
#endif
constexpr int kTopkNT = MOE_TOPK_NT;                    // tokens ranked side by side per wavefront
constexpr int kTopkThreads = kChunk / kTopkNT * 64;      // one token group per wavefront
// Threads of a top-k block: the 16-lane group layout holds one chunk in 8
// wavefronts; the other layouts one chunk in 16.
constexpr int topk_threads(int GL) { return GL == 16 ? 512 : kTopkThreads; }

// Tokens a wavefront ranks side by side in the filter: two while their
// registers leave room for two blocks per CU, else one after the other.
template <int CPL>
constexpr int topk_filter_nt() { return CPL >= 16 ? 1 : 2; }

template <int CPL>
MOE_DEV void topk_block(int chunk, uint32_t* mask, float* sb, TopkScratch* scratch, const float* __restrict__ logits,
                        const float* __restrict__ bias, int T, int E, int k, float scale, int32_t* __restrict__ idx,
                        float* __restrict__ gates, uint32_t* __restrict__ bitmap, int32_t* __restrict__ ssum) {
  constexpr int NW = kChunk / kTopkNT;
  constexpr int NF = topk_filter_nt<CPL>();
  static_assert(kTopkNT % NF == 0, "filter groups tile a wavefront's tokens");
  for (int i = threadIdx.x; i < E; i += kTopkThreads) {
    mask[i] = 0u;
    sb[i] = bias[i];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  TopkScratch* ts = scratch + wave * kTopkNT;
  int t[kTopkNT];
  int n = 0;
#pragma unroll
  for (int u = 0; u < kTopkNT; ++u) {
    t[u] = chunk * kChunk + wave + NW * u;
    n += t[u] < T;
  }
  bool fb[kTopkNT];
  if (n == kTopkNT) {
#pragma unroll
    for (int u0 = 0; u0 < kTopkNT; u0 += NF) {
      int tg[NF];
      bool fg[NF];
#pragma unroll
      for (int u = 0; u < NF; ++u) tg[u] = t[u0 + u];
      topk_filter_tokens<CPL, NF>(logits, sb, tg, E, k, scale, idx, gates, mask, ts + u0, fg);
#pragma unroll
      for (int u = 0; u < NF; ++u) fb[u0 + u] = fg[u];
    }
  } else {
    for (int u = 0; u < kTopkNT; ++u) fb[u] = false;
    for (int u = 0; u < n; ++u) {  // ragged last chunk: one at a time
      const int t1[1] = {t[u]};
      bool f1[1];
      topk_filter_tokens<CPL, 1>(logits, sb, t1, E, k, scale, idx, gates, mask, ts, f1);
      fb[u] = f1[0];
    }
  }
  bool any = false;
#pragma unroll
  for (int u = 0; u < kTopkNT; ++u) any |= fb[u];
  if (any) {  // tokens with too many candidates: the k-round selection
    for (int u = 0; u < kTopkNT; ++u)
      if (fb[u]) {
        const int t1[1] = {t[u]};
        topk_tokens<CPL, 1>(logits, sb, t1, E, k, scale, idx, gates, mask);
      }
  }
  __syncthreads();
  // the chunk's masks, and its counts added to its super-chunk's totals
  // (integer atomics: the sums do not depend on the order of the chunks)
  int32_t* sdst = ssum + (size_t)(chunk / kSuper) * E;
  for (int i = threadIdx.x; i < E; i += kTopkThreads) {
    const uint32_t m = mask[i];
    bitmap[(size_t)chunk * E + i] = m;
    if (m) atomicAdd(&sdst[i], __popc(m));
  }
}

// Group layout for E <= 16 GL and k <= GL / 2: a token per group of GL = 16
// lanes (a DPP row; four tokens per wavefront) or 32 lanes (two per
// wavefront), so the per-token steps (threshold, exact scores, ranking,
// gates) are shared by the wavefront's tokens.  Lane li of a group holds
// experts li + GL c; the groups of the threshold are the GL lanes of the
// token (GL >= 2k); at most GL candidates per token (one per lane of its
// group), else that token takes the k-round path.  Same result as
// topk_tokens, bit for bit.
template <int GL>
constexpr int group_max_k() { return GL / 2; }

// Inclusive prefix (sum, or minimum with MIN) over the GL lanes of each group:
// DPP row shifts within 16-lane rows, then one shuffle across the two rows of
// a 32-lane group.
template <int GL, bool MIN>
MOE_DEV int32_t group_scan(int32_t v) {
  const int32_t id = MIN ? INT32_MAX : 0;
  auto op = [](int32_t a, int32_t b) { return MIN ? min(a, b) : a + b; };
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xF, 0xF, false));
  if constexpr (GL == 32) {
    const int32_t u = __shfl(v, (threadIdx.x & 32) | 15, 64);  // the lower row's last value
    if (threadIdx.x & 16) v = op(v, u);
  }
  return v;
}

template <int GL>
MOE_DEV int32_t group_last(int32_t v) { return __shfl(v, (threadIdx.x & (64 - GL)) | (GL - 1), 64); }

template <int CPR, int GL>
MOE_DEV bool topk_group_tokens(const float* __restrict__ logits, const float* sb, const float* sbt, int t,
                               bool valid, int E, int k, float scale, int32_t* __restrict__ idx,
                               float* __restrict__ gates, uint32_t* mask, TopkScratch* ws) {
#pragma clang fp contract(off)
  constexpr int BV = CPR % 4 == 0 ? 4 : CPR % 2 == 0 ? 2 : 1;  // bias columns per LDS read
  const int lane = threadIdx.x & 63, li = lane & (GL - 1), rb = lane & (64 - GL);
  float l[CPR];
  int32_t q[CPR];
  int32_t mx = INT32_MIN;
  // branch-free loads: rows past T and columns past E read a valid element,
  // whose key is replaced below
  const float* lr = logits + (size_t)(valid ? t : 0) * E;
#pragma unroll
  for (int c = 0; c < CPR; ++c) l[c] = lr[min(li + GL * c, E - 1)];
#pragma unroll
  for (int c0 = 0; c0 < CPR; c0 += BV) {
    // the lane's bias columns, BV per LDS read (sbt[li][c] = b[li + GL c])
    float bc[BV];
    if constexpr (BV == 4) {
      const float4 b4 = *reinterpret_cast<const float4*>(sbt + li * CPR + c0);
      bc[0] = b4.x, bc[1] = b4.y, bc[2] = b4.z, bc[3] = b4.w;
    } else if constexpr (BV == 2) {
      const float2 b2 = *reinterpret_cast<const float2*>(sbt + li * CPR + c0);
      bc[0] = b2.x, bc[1] = b2.y;
    } else {
      bc[0] = sbt[li * CPR + c0];
    }
#pragma unroll
    for (int u = 0; u < BV; ++u) {
      const int c = c0 + u, e = li + GL * c;
      const int32_t key = float_skey(fast_sigmoid(l[c]) + bc[u]);
      q[c] = (valid && e < E) ? key : INT32_MIN;
      mx = max(mx, q[c]);
    }
  }
  ws->m[lane] = mx;
  wave_lds_sync();
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < GL; i += 4) {
    const int4 w = *reinterpret_cast<const int4*>(&ws->m[rb + i]);
    cnt += (w.x > mx) + (w.y > mx) + (w.z > mx) + (w.w > mx);
  }
  // the group's smallest lane maximum with fewer than k larger ones
  const int32_t tau = group_last<GL>(group_scan<GL, true>(cnt < k ? mx : INT32_MAX));
  const float vt = skey_float(tau);
  const int32_t thr = __builtin_isfinite(vt) ? float_skey(vt - (0x1p-12f + fabsf(vt) * 0x1p-16f)) : INT32_MIN + 1;
  // compaction: each lane's candidates after those of the lanes before it in the group
  int n = 0;
#pragma unroll
  for (int c = 0; c < CPR; ++c) n += q[c] >= thr;
  const int incl = group_scan<GL, false>(n);
  const int C = group_last<GL>(incl);
  const bool fb = valid && (C < k || C > GL);
  const bool act = valid && !fb;
  if (act) {
    int pos = rb + incl - n;
#pragma unroll
    for (int c = 0; c < CPR; ++c)
      if (q[c] >= thr) {
        ws->cl[pos] = l[c];
        ws->ce[pos] = li + GL * c;
        ++pos;
      }
  }
  wave_lds_sync();
  const bool mine = act && li < C;  // this lane scores candidate li of its group
  float sv = 0.f;
  int ev = 0;
  unsigned long long R = 0ull;
  if (mine) {
    ev = ws->ce[lane];
    sv = router_sigmoid(ws->cl[lane]);
    R = ((unsigned long long)float_order_key(sv + sb[ev]) << 32) | (uint32_t)~ev;
  }
  ws->r[lane] = R;  // zero past the candidates: below every real key
  wave_lds_sync();
  const int cw = act ? C : 0;
  int cmax = 0;
#pragma unroll
  for (int g = 0; g < 64 / GL; ++g) cmax = max(cmax, __builtin_amdgcn_readlane(cw, g * GL + GL - 1));
  int rank = 0;
  for (int i = 0; i < cmax; i += 2) {
    const ulonglong2 w = *reinterpret_cast<const ulonglong2*>(&ws->r[rb + i]);
    rank += (w.x > R) + (w.y > R);
  }
  wave_lds_sync();
  if (mine && rank < k) ws->m[rb + rank] = __float_as_int(sv);
  wave_lds_sync();
  if (mine && rank < k) {
    float S = __int_as_float(ws->m[rb]);  // the gates' denominator: fp32 sum in slot order
    for (int j = 1; j < k; ++j) S = S + __int_as_float(ws->m[rb + j]);
    const size_t o = (size_t)t * k + rank;
    idx[o] = ev;
    gates[o] = (sv / S) * scale;
    atomicOr(&mask[ev], 1u << (t & 31));
  }
  wave_lds_sync();
  return fb;
}

// Block of the group layout: one chunk, GL / 2 wavefronts (8 for GL = 16,
// 16 for GL = 32) of 64 / GL tokens each.  One chunk per block keeps the
// block barriers to the wavefronts of one chunk and, for GL = 16, gives four
// resident blocks per CU instead of two (decode shape, T = 131072: 44.8 ->
// 42.1 us frozen, 80.0 -> 73.5 us in training with twice the histogram
// parts).
template <int CPL, int GL>
MOE_DEV void topk_group_block(int blk, uint32_t* maskc, float* sb, TopkScratch* scratch,
                              const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
                              float scale, int32_t* __restrict__ idx, float* __restrict__ gates,
                              uint32_t* __restrict__ bitmap, int32_t* __restrict__ ssum, int nchunks) {
  constexpr int CPR = 64 * CPL / GL, WPC = GL / 2, TPW = 64 / GL, NTHR = topk_threads(GL);
  constexpr int NCH = NTHR / 64 / WPC;  // chunks per block
  static_assert(NCH >= 1 && NTHR == NCH * WPC * 64, "whole chunks per block");
  static_assert(GL * CPR <= 512, "the lane-major bias copy fits beside the bias");
  float* sbt = sb + 512;  // sbt[li * CPR + c] = bias[li + GL c] (0 past E)
  for (int i = threadIdx.x; i < E; i += NTHR) {
#pragma unroll
    for (int h = 0; h < NCH; ++h) maskc[h * E + i] = 0u;
    sb[i] = bias[i];
  }
  for (int i = threadIdx.x; i < GL * CPR; i += NTHR) sbt[(i % GL) * CPR + i / GL] = i < E ? bias[i] : 0.f;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = wave / WPC;                   // which chunk of the block
  const int chunk = NCH * blk + half;
  uint32_t* mask = maskc + half * E;
  const int t0 = chunk * kChunk + (wave % WPC) * TPW;
  const int t = t0 + lane / GL;
  const bool valid = chunk < nchunks && t < T;
  const bool fb = topk_group_tokens<CPR, GL>(logits, sb, sbt, t, valid, E, k, scale, idx, gates, mask, scratch + wave);
  const unsigned long long fbm = __ballot(fb && (lane & (GL - 1)) == 0);
  for (int r = 0; r < TPW; ++r)  // tokens with more than GL candidates: the k-round selection
    if ((fbm >> (GL * r)) & 1ull) {
      const int t1[1] = {t0 + r};
      topk_tokens<CPL, 1>(logits, sb, t1, E, k, scale, idx, gates, mask);
    }
  __syncthreads();
  for (int hh = 0; hh < NCH; ++hh) {
    const int c = NCH * blk + hh;
    if (c >= nchunks) break;
    int32_t* sdst = ssum + (size_t)(c / kSuper) * E;
    for (int i = threadIdx.x; i < E; i += NTHR) {
      const uint32_t m = maskc[hh * E + i];
      bitmap[(size_t)c * E + i] = m;
      if (m) atomicAdd(&sdst[i], __popc(m));
    }
  }
}

// ---------------------------------------------------------- QB histogram ----
// The state keeps one histogram [E][B].  Block (16-expert group, token part)
// counts its part's score bins in LDS with integer atomics and adds them to
// the histogram rows with global integer atomics: both are order-free, so the
// histogram is the same whatever order the blocks run in.
template <int NTHR>
MOE_DEV void hist_block(int group, int ts, uint32_t* lh, const float* __restrict__ logits, int T, int E, int B,
                        float lo, float scale, int tps, uint32_t* __restrict__ hist,
                        unsigned long long* __restrict__ count) {
  constexpr int TR = NTHR / kHistExperts;  // token rows in flight per step
  const int e0 = group * kHistExperts;
  const int ne = min(kHistExperts, E - e0);
  const int nb = kHistExperts * B;
  for (int i = threadIdx.x; i < nb; i += NTHR) lh[i] = 0;
  __syncthreads();
  // thread -> expert e0 + (i % 16), tokens (i / 16) + TR m: each wavefront
  // reads four 64-byte row pieces per step
  const int el = threadIdx.x % kHistExperts, tl = threadIdx.x / kHistExperts;
  const int e = e0 + el;
  const int tb = ts * tps, te = min(T, tb + tps);
  if (e < E) {
    uint32_t* row = lh + el * B;
    int t = tb + tl;
    for (; t + TR < te; t += 2 * TR) {
      const float l0 = logits[(size_t)t * E + e], l1 = logits[(size_t)(t + TR) * E + e];
      atomicAdd(&row[score_bin_fast(l0, B, lo, scale)], 1u);
      atomicAdd(&row[score_bin_fast(l1, B, lo, scale)], 1u);
    }
    for (; t < te; t += TR)
      atomicAdd(&row[score_bin_fast(logits[(size_t)t * E + e], B, lo, scale)], 1u);
  }
  __syncthreads();
  if (tb < T) {  // integer atomics: the sums do not depend on the order of the token parts
    uint32_t* dst = hist + (size_t)e0 * B;
    for (int i = threadIdx.x; i < ne * B; i += NTHR) {
      const uint32_t v = lh[i];
      if (v) atomicAdd(&dst[i], v);
    }
  }
  if (group == 0 && ts == 0 && threadIdx.x == 0) *count += (unsigned long long)T;
}

// One launch for the scores: the last blocks rank the chunks; in
// training mode the blocks before them build the QB histogram from the same
// logits (independent work side by side instead of two launches; the fewer,
// longer histogram blocks are dispatched first so that they overlap the
// ranking instead of trailing it).
template <int CPL, int GL>
__global__ __launch_bounds__(topk_threads(GL)) __attribute__((amdgpu_waves_per_eu(8))) void k_topk(const float* __restrict__ logits,
                                                       const float* __restrict__ bias, int T, int E, int k,
                                                       float scale, int32_t* __restrict__ idx,
                                                       float* __restrict__ gates, uint32_t* __restrict__ bitmap,
                                                       int nchunks, int B, float lo, float bscale, int tps,
                                                       uint32_t* __restrict__ hist,
                                                       unsigned long long* __restrict__ count,
                                                       int32_t* __restrict__ ssum) {
  // masks, bias, exchange (one TopkScratch per token group: per wavefront in
  // the group layout, kTopkNT per wavefront in the 64-lane one)
  constexpr int kScratches = GL ? topk_threads(GL) / 64 : kChunk;
  constexpr int kTopkBytes = 2 * 1024 * 4 + kScratches * (int)sizeof(TopkScratch);
  constexpr int kHistBytes = kHistExperts * 256 * 4;
  __shared__ __align__(16) uint32_t smem[(kTopkBytes > kHistBytes ? kTopkBytes : kHistBytes) / 4];
  const int nrank = nchunks;  // one chunk per ranking block
  const int nhist = (int)gridDim.x - nrank;
  if ((int)blockIdx.x >= nhist) {
    if constexpr (GL != 0)
      topk_group_block<CPL, GL>(blockIdx.x - nhist, smem, reinterpret_cast<float*>(smem + 1024),
                                reinterpret_cast<TopkScratch*>(smem + 2048), logits, bias, T, E, k, scale, idx,
                                gates, bitmap, ssum, nchunks);
    else
      topk_block<CPL>(blockIdx.x - nhist, smem, reinterpret_cast<float*>(smem + 1024),
                      reinterpret_cast<TopkScratch*>(smem + 2048), logits, bias, T, E, k, scale, idx, gates, bitmap,
                      ssum);
  } else {
    const int groups = (E + kHistExperts - 1) / kHistExperts;
    hist_block<topk_threads(GL)>(blockIdx.x % groups, blockIdx.x / groups, smem, logits, T, E, B, lo, bscale, tps,
                                 hist, count);
  }
}

// Lanes per token of the group layout (0: the 64-lane layout).  A group of
// GL lanes holds 64 CPL / GL <= 16 columns and ranks up to GL / 2 experts.
// Up to 512 chunks (16384 tokens) 32 lanes per token give half the columns
// per lane and, with a chunk per block either way, twice the lanes per block
// (replica, T = 8192: 11.3 -> 9.6 us against 16 lanes); beyond that 16 lanes,
// sharing the per-token steps four ways, are faster (decode, T = 131072: 49
// against 59 us when measured).
static int topk_group_lanes(int cpl, int k, int nchunks) {
  const bool g16 = cpl <= 4 && k <= group_max_k<16>(), g32 = cpl <= 8 && k <= group_max_k<32>();
  if (g16 && nchunks > 512) return 16;
  return g32 ? 32 : g16 ? 16 : 0;
}

hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       uint32_t* bitmap, uint32_t* hist, unsigned long long* count, int32_t* ssum, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cpl = (D.E + 63) / 64;
  const int gl = topk_group_lanes(cpl, D.k, nchunks);
  // token parts of the histogram: kHistParts per 1024 threads a block has, so
  // smaller blocks keep the same threads on it; half as many in the 64-lane
  // layout (large E), whose many expert groups otherwise outnumber the ranking
  // blocks (k3 shape: 48.4 -> 43.9 us in training; a quarter, or half at the
  // replica shape, were slower)
  const int parts = gl ? kHistParts * kTopkThreads / topk_threads(gl) : kHistParts / 2;
  const int tps = (T + parts - 1) / parts;
  const int hblocks = hist ? (D.E + kHistExperts - 1) / kHistExperts * parts : 0;
  dim3 grid(nchunks + hblocks), block(topk_threads(gl));
#define MOE_TOPK(C, G)                                                                                          \
  hipLaunchKernelGGL((k_topk<C, G>), grid, block, 0, s, logits, bias, T, D.E, D.k, D.routed_scale, idx, gates, \
                     bitmap, nchunks, D.B, D.qb_lo, D.qb_scale, tps, hist, count, ssum)
  if (cpl <= 1) { if (gl == 16) MOE_TOPK(1, 16); else if (gl == 32) MOE_TOPK(1, 32); else MOE_TOPK(1, 0); }
  else if (cpl <= 2) { if (gl == 16) MOE_TOPK(2, 16); else if (gl == 32) MOE_TOPK(2, 32); else MOE_TOPK(2, 0); }
  else if (cpl <= 4) { if (gl == 16) MOE_TOPK(4, 16); else if (gl == 32) MOE_TOPK(4, 32); else MOE_TOPK(4, 0); }
  else if (cpl <= 8) { if (gl == 32) MOE_TOPK(8, 32); else MOE_TOPK(8, 0); }
  else MOE_TOPK(16, 0);
#undef MOE_TOPK
  return hipGetLastError();
}

// ------------------------------------------------------- counts / scan ----
// Two-level exclusive prefix sums of the per-(chunk, expert) selection counts
// popcount(bitmap[c][e]).  The top-k launch leaves each super-chunk's (kSuper
// chunks') total per expert in sbase; the global scan below turns those into
// first rows; the base of a chunk inside its super-chunk is summed by the
// scatter from the masks themselves.
// At most 8 tiles of kExpertBM rows per expert on average: the scan's one
// thread per expert writes that expert's tiles; otherwise the scatter launch
// writes the tile tables, spread over its blocks.
__host__ __device__ inline bool scan_writes_tiles(int T, int k, int E) {
  return (long long)T * k <= 8LL * kExpertBM * E;
}

// Super-chunks [s0, s1) of expert e: each total in sbase becomes the first
// row of its part of the expert's group, counting on from `run` (16 loads
// issued before their stores: the compiler cannot tell that the stores do
// not alias the next loads).
MOE_DEV void prefix_rows(int32_t* __restrict__ sbase, int E, int e, int s0, int s1, int run) {
  for (int sc0 = s0; sc0 < s1; sc0 += 16) {
    int x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = sc0 + u < s1 ? sbase[(size_t)(sc0 + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (sc0 + u < s1) {
        sbase[(size_t)(sc0 + u) * E + e] = run;
        run += x[u];
      }
  }
}

// Global (one block of 1024 threads, one expert per thread, or several when
// there are more super-chunks than registers and few experts): per expert, the
// total and the exclusive prefix over super-chunks (sbase becomes the
// absolute first row of each super-chunk's part of the expert's group); over
// experts, the row offsets and the first m-tile of each expert for the grouped
// GEMMs (tiles of kExpertBM rows; an empty expert has none).  With `load`
// (sign-rule training) each expert's count is added to its accumulated load
// and T to the token count.
__global__ __launch_bounds__(1024) void k_scan_global(int32_t* __restrict__ sbase, int nsuper, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ tile_offsets, int2* __restrict__ tile_info,
                                                      uint32_t* __restrict__ load, unsigned long long* __restrict__ count,
                                                      int T, int k, int32_t* __restrict__ tile_offsets2,
                                                      int2* __restrict__ tile_info2) {
  __shared__ int wsum_r[16], wsum_t[16], wsum_u[16];
  __shared__ int s_row0[1024];  // per expert (E <= 1024): first row
  __shared__ int s_part[1024];  // many super-chunks: each thread's partial sum
  constexpr int kReg = 16;  // up to this many super-chunk totals stay in registers
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  const bool few = scan_writes_tiles(T, k, E);
  // More super-chunks than registers and E <= 512: P threads per expert
  // (P E <= 1024), thread i takes expert i % E and the P-th part i / E of its
  // super-chunks, so that P times more loads are in flight.
  int P = 1;
  while (2 * P * E <= 1024) P *= 2;
  const bool split = nsuper > kReg && P > 1;
  const int part = i / E, pe = i - part * E;
  const int pm = (nsuper + P - 1) / P, ps0 = min(nsuper, part * pm), ps1 = min(nsuper, ps0 + pm);
  int c = 0;
  int v[kReg];
  if (!split) {
    if (i < E) {
      if (nsuper <= kReg) {
#pragma unroll
        for (int sc = 0; sc < kReg; ++sc) {
          v[sc] = sc < nsuper ? sbase[(size_t)sc * E + i] : 0;
          c += v[sc];
        }
      } else {
#pragma unroll 16
        for (int sc = 0; sc < nsuper; ++sc) c += sbase[(size_t)sc * E + i];
      }
    }
  } else {
    int ps = 0;
    if (part < P) {
#pragma unroll 16
      for (int sc = ps0; sc < ps1; ++sc) ps += sbase[(size_t)sc * E + pe];
    }
    s_part[i] = ps;
    __syncthreads();
    if (i < E)
      for (int q = 0; q < P; ++q) c += s_part[q * E + i];
  }
  const int tl = (c + kExpertBM - 1) / kExpertBM, tl2 = (c + kExpertBM2 - 1) / kExpertBM2;
  int r = c, t = tl, u = tl2;  // inclusive wave scans
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ro = __shfl_up(r, o, 64), to = __shfl_up(t, o, 64), uo = __shfl_up(u, o, 64);
    if (lane >= o) {
      r += ro;
      t += to;
      u += uo;
    }
  }
  if (lane == 63) {
    wsum_r[w] = r;
    wsum_t[w] = t;
    wsum_u[w] = u;
  }
  __syncthreads();
  for (int j = 0; j < w; ++j) {
    r += wsum_r[j];
    t += wsum_t[j];
    u += wsum_u[j];
  }
  if (i < E) {
    counts[i] = c;
    if (load) load[i] += (uint32_t)c;
    offsets[i + 1] = r;
    tile_offsets[i + 1] = t;
    int run = r - c;  // exclusive offset of expert i
    if (nsuper <= kReg) {
#pragma unroll
      for (int sc = 0; sc < kReg; ++sc) {
        if (sc < nsuper) sbase[(size_t)sc * E + i] = run;
        run += v[sc];
      }
    } else if (!split) {
      prefix_rows(sbase, E, i, 0, nsuper, run);
    }
    s_row0[i] = r - c;
    if (tile_offsets2) tile_offsets2[i + 1] = u;
    if (few) {  // each expert thread writes its own few tiles
      for (int j = 0, t0 = t - tl; j < tl; ++j)
        tile_info[t0 + j] = make_int2(r - c + j * kExpertBM, (i << 8) | min(kExpertBM, c - j * kExpertBM));
      if (tile_info2)
        for (int j = 0, u0 = u - tl2; j < tl2; ++j)
          tile_info2[u0 + j] = make_int2(r - c + j * kExpertBM2, (i << 8) | min(kExpertBM2, c - j * kExpertBM2));
    }
  }
  if (i == 0) {
    offsets[0] = 0;
    tile_offsets[0] = 0;
    if (tile_offsets2) tile_offsets2[0] = 0;
    if (load) *count += (unsigned long long)T;
  }
  if (split) {
    __syncthreads();
    if (part < P) {  // each part's super-chunks become first rows, from its base
      int run = s_row0[pe];
      for (int q = 0; q < part; ++q) run += s_part[q * E + pe];
      prefix_rows(sbase, E, pe, ps0, ps1, run);
    }
  }
  // many tiles per expert: the scatter launch writes the tile tables
}

hipError_t launch_scan(const Dims& D, int T, int32_t* sbase, int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                       int2* tile_info, uint32_t* load, unsigned long long* count, hipStream_t s,
                       int32_t* tile_offsets2, int2* tile_info2) {
  if ((tile_offsets2 == nullptr) != (tile_info2 == nullptr)) return hipErrorInvalidValue;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int nsuper = (nchunks + kSuper - 1) / kSuper;
  hipLaunchKernelGGL(k_scan_global, dim3(1), dim3(1024), 0, s, sbase, nsuper, D.E, counts, offsets, tile_offsets,
                     tile_info, load, load ? count : nullptr, T, D.k, tile_offsets2, tile_info2);
  return hipGetLastError();
}

// -------------------------------------------------------------- scatter ----
// Stable rows without order-dependent atomics: the row of (t, j) in expert
// e's group is the super-chunk's first row (global scan) + the tokens of e in
// the earlier chunks of the super-chunk (their masks' popcounts) + the
// earlier tokens of the chunk in the chunk's mask for e.  Two launch forms:
// one thread per (t, j) summing those popcounts itself (at most kSuper - 1
// mask loads, all in flight together), and, for long batches with E <= 256,
// one block per kWideG chunks that forms every expert's chunk first rows once
// (whole mask rows, coalesced across the experts) and keeps them with the
// chunk masks in LDS, so each (t, j) loads only its expert index (decode
// shape, T = 131072: 19.8 -> 14 us; below 2048 chunks the per-(t, j) form is
// faster).
// Tile table entries (many tiles per expert): tile g belongs to the first
// expert e with pre[e] > g, pre the inclusive tile prefix (tile_offsets[1 ..
// E]), found by a binary search over a copy of pre in LDS; consecutive
// entries per wavefront, so the stores coalesce (a grid-stride loop: every
// table has at most T k tiles, each holding at least one row).
MOE_DEV void fill_tiles(int* s_pre, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                        const int32_t* __restrict__ tile_offsets, int2* __restrict__ info, int bm, int E,
                        int grid_threads) {
  const int total = tile_offsets[E];
  if ((int)blockIdx.x * 256 >= total) return;  // block-uniform
  for (int i = threadIdx.x; i < E; i += 256) s_pre[i] = tile_offsets[i + 1];
  __syncthreads();
  for (int g = blockIdx.x * 256 + threadIdx.x; g < total; g += grid_threads) {
    int lo = 0, hi = E - 1;  // first e with pre[e] > g
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] > g) hi = mid;
      else lo = mid + 1;
    }
    const int j = g - (lo > 0 ? s_pre[lo - 1] : 0), c = counts[lo];
    info[g] = make_int2(offsets[lo] + j * bm, (lo << 8) | min(bm, c - j * bm));
  }
  __syncthreads();  // s_pre is reused next
}

struct ScatterArgs {
  const int32_t* idx;
  const uint32_t* bitmap;
  const int32_t* sbase;
  int32_t* perm_src;
  int32_t* inv;
  const uint32_t* zs;  // block-scaled experts: each token's scale row (s4 words), copied to its grouped rows
  uint32_t* Xs;
  int s4;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tile_offsets;
  int2* tile_info;  // NULL: the scan wrote the tile tables
  const int32_t* tile_offsets2;
  int2* tile_info2;
};

MOE_DEV void fill_tables(int* s_pre, const ScatterArgs& a, int E, int grid_threads) {
  if (a.tile_info) {
    fill_tiles(s_pre, a.counts, a.offsets, a.tile_offsets, a.tile_info, kExpertBM, E, grid_threads);
    if (a.tile_info2)
      fill_tiles(s_pre, a.counts, a.offsets, a.tile_offsets2, a.tile_info2, kExpertBM2, E, grid_threads);
  }
}

MOE_DEV void place(const ScatterArgs& a, int p, int t, int row, int Tk) {
  a.inv[p] = row;
  if ((unsigned)row < (unsigned)Tk) {  // always true for a consistent permutation
    a.perm_src[row] = t;
    for (int q = 0; q < a.s4; ++q) a.Xs[(size_t)row * a.s4 + q] = a.zs[(size_t)t * a.s4 + q];
  }
}

__global__ __launch_bounds__(256) void k_scatter(ScatterArgs a, int T, int E, int k, int grid_threads) {
  __shared__ int s_pre[1024];
  fill_tables(s_pre, a, E, grid_threads);
  const int Tk = T * k;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= Tk) return;
  const int t = p / k;
  const int e = a.idx[p];
  const int c = t / kChunk, c0 = c - c % kSuper;
  uint32_t m[kSuper - 1];
#pragma unroll
  for (int j = 0; j < kSuper - 1; ++j) m[j] = c0 + j < c ? a.bitmap[(size_t)(c0 + j) * E + e] : 0u;
  int cb = 0;
#pragma unroll
  for (int j = 0; j < kSuper - 1; ++j) cb += __popc(m[j]);
  const uint32_t below = a.bitmap[(size_t)c * E + e] & ((1u << (t % kChunk)) - 1u);
  place(a, p, t, a.sbase[(size_t)(c / kSuper) * E + e] + cb + __popc(below), Tk);
}

constexpr int kWideG = 8;  // chunks per block of the wide form (divides kSuper)
constexpr int kWidePre = 8;  // expert indices per thread loaded before the masks
static_assert(kSuper % kWideG == 0 && kSuper - kWideG <= 8, "one batch of earlier mask rows");

__global__ __launch_bounds__(256) void k_scatter_wide(ScatterArgs a, int T, int E, int k, int grid_threads) {
  __shared__ int s_row[kWideG * 256];        // [chunk][expert] first rows
  __shared__ uint32_t s_mask[kWideG * 256];  // [chunk][expert] masks
  fill_tables(s_row, a, E, grid_threads);
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cb = blockIdx.x * kWideG, c0 = cb - cb % kSuper, cn = min(kWideG, nchunks - cb);
  const int Tk = T * k, pb = cb * kChunk * k, p1 = min(T, (cb + cn) * kChunk) * k;
  int ep[kWidePre];
#pragma unroll
  for (int u = 0; u < kWidePre; ++u) {
    const int p = pb + (int)threadIdx.x + 256 * u;
    ep[u] = p < p1 ? a.idx[p] : 0;
  }
  const int e = threadIdx.x;
  if (e < E) {
    uint32_t me[kSuper - kWideG], mo[kWideG];
#pragma unroll
    for (int u = 0; u < kSuper - kWideG; ++u) me[u] = c0 + u < cb ? a.bitmap[(size_t)(c0 + u) * E + e] : 0u;
#pragma unroll
    for (int u = 0; u < kWideG; ++u) mo[u] = u < cn ? a.bitmap[(size_t)(cb + u) * E + e] : 0u;
    int run = a.sbase[(size_t)(cb / kSuper) * E + e];
#pragma unroll
    for (int u = 0; u < kSuper - kWideG; ++u) run += __popc(me[u]);
#pragma unroll
    for (int u = 0; u < kWideG; ++u) {
      s_row[u * 256 + e] = run;
      s_mask[u * 256 + e] = mo[u];
      run += __popc(mo[u]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kWidePre; ++u) {
    const int p = pb + (int)threadIdx.x + 256 * u;
    if (p < p1) {
      const int t = p / k, g = t / kChunk - cb, ee = ep[u];
      const uint32_t below = s_mask[g * 256 + ee] & ((1u << (t % kChunk)) - 1u);
      place(a, p, t, s_row[g * 256 + ee] + __popc(below), Tk);
    }
  }
  for (int p = pb + kWidePre * 256 + (int)threadIdx.x; p < p1; p += 256) {
    const int t = p / k, g = t / kChunk - cb, ee = a.idx[p];
    const uint32_t below = s_mask[g * 256 + ee] & ((1u << (t % kChunk)) - 1u);
    place(a, p, t, s_row[g * 256 + ee] + __popc(below), Tk);
  }
}

hipError_t launch_scatter(const Dims& D, const int32_t* idx, const uint32_t* bitmap, const int32_t* sbase, int T,
                          int32_t* perm_src, int32_t* inv, hipStream_t s, const uint8_t* zs, uint8_t* Xs, int s_ld,
                          const int32_t* counts, const int32_t* offsets, const int32_t* tile_offsets,
                          int2* tile_info, const int32_t* tile_offsets2, int2* tile_info2) {
  const long long Tk = (long long)T * D.k;
  if (zs && s_ld % 4) return hipErrorInvalidValue;
  if ((tile_offsets2 == nullptr) != (tile_info2 == nullptr)) return hipErrorInvalidValue;
  const bool fill = !scan_writes_tiles(T, D.k, D.E);  // else the scan wrote them
  if (fill && (!counts || !offsets || !tile_offsets || !tile_info)) return hipErrorInvalidValue;
  const ScatterArgs a{idx, bitmap, sbase, perm_src, inv, reinterpret_cast<const uint32_t*>(zs),
                      reinterpret_cast<uint32_t*>(Xs), zs ? s_ld / 4 : 0, counts, offsets, tile_offsets,
                      fill ? tile_info : nullptr, tile_offsets2, fill ? tile_info2 : nullptr};
  const int nchunks = (T + kChunk - 1) / kChunk;
  // the fill's stride, the grid's thread count, comes as an argument
  if (nchunks > 2048 && D.E <= 256) {
    const unsigned blocks = (unsigned)((nchunks + kWideG - 1) / kWideG);
    hipLaunchKernelGGL(k_scatter_wide, dim3(blocks), dim3(256), 0, s, a, T, D.E, D.k, (int)blocks * 256);
  } else {
    const unsigned blocks = (unsigned)((Tk + 255) / 256);
    hipLaunchKernelGGL(k_scatter, dim3(blocks), dim3(256), 0, s, a, T, D.E, D.k, (int)blocks * 256);
  }
  return hipGetLastError();
}

// -------------------------------------------------------------- combine ----
// y_lat[t] = sum_j g[t,j] Y[inv[t,j]] in slot order, fp32, stored in the
// activation dtype.  One wavefront per token; lane c handles 4 latent
// columns per 4*64-column stripe, with the row loads of up to 8 slots in
// flight before they are summed (in slot order).
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ Y, const float* __restrict__ gates,
                                                 const int32_t* __restrict__ inv, int T, int l, int k,
                                                 void* __restrict__ y_lat) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = 0;
  float my_g = 0.f;
  if (lane < k) {
    my_row = inv[(size_t)t * k + lane];
    my_g = gates[(size_t)t * k + lane];
    if ((unsigned)my_row >= (unsigned)(T * k)) my_row = 0;  // never taken for a consistent permutation
  }
  const int nq = l / 4;  // groups of 4 columns
  constexpr int J = 8;   // slots whose row loads are in flight together
  for (int q = lane; q < nq; q += 64) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j0 = 0; j0 < k; j0 += J) {
      // readlane, not a shuffle: lanes past l/4 are inactive in this loop
      if (BF16) {
        uint2 v[J];
#pragma unroll
        for (int u = 0; u < J; ++u)
          if (j0 + u < k) {
            const int row = __builtin_amdgcn_readlane(my_row, j0 + u);
            v[u] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(Y) + (size_t)row * l + 4 * q);
          }
#pragma unroll
        for (int u = 0; u < J; ++u)
          if (j0 + u < k) {
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j0 + u));
            a0 += g * bf16_bits_to_f32(v[u].x & 0xFFFFu);
            a1 += g * bf16_bits_to_f32(v[u].x >> 16);
            a2 += g * bf16_bits_to_f32(v[u].y & 0xFFFFu);
            a3 += g * bf16_bits_to_f32(v[u].y >> 16);
          }
      } else {
        float4 v[J];
#pragma unroll
        for (int u = 0; u < J; ++u)
          if (j0 + u < k) {
            const int row = __builtin_amdgcn_readlane(my_row, j0 + u);
            v[u] = *reinterpret_cast<const float4*>(static_cast<const float*>(Y) + (size_t)row * l + 4 * q);
          }
#pragma unroll
        for (int u = 0; u < J; ++u)
          if (j0 + u < k) {
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j0 + u));
            a0 += g * v[u].x;
            a1 += g * v[u].y;
            a2 += g * v[u].z;
            a3 += g * v[u].w;
          }
      }
    }
    if (BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y_lat) + (size_t)t * l + 4 * q) =
          make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(y_lat) + (size_t)t * l + 4 * q) = make_float4(a0, a1, a2, a3);
    }
  }
}

// bf16 rows of l = 64 CW columns: lane c takes CW consecutive columns, so one
// wavefront load covers whole rows (2 KB at l = 1024) instead of 512-byte
// pieces in separate batches; the row loads of J = 8 / (CW / 8) slots are in
// flight together.  Same slot-order fp32 sums as k_combine (k3 shape, l =
// 1024, k = 16: 117.2 -> 114.5 us; the gathered reads stay bound by HBM's
// random-access rate).
template <int CW>
__global__ __launch_bounds__(256) void k_combine_wide(const uint16_t* __restrict__ Y, const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int T, int k,
                                                      uint16_t* __restrict__ y_lat) {
  constexpr int NC = CW / 8, J = 8 / NC, l = 64 * CW;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = 0;
  float my_g = 0.f;
  if (lane < k) {
    my_row = inv[(size_t)t * k + lane];
    my_g = gates[(size_t)t * k + lane];
    if ((unsigned)my_row >= (unsigned)(T * k)) my_row = 0;  // never taken for a consistent permutation
  }
  float a[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) a[c] = 0.f;
  for (int j0 = 0; j0 < k; j0 += J) {
    uint4 v[J][NC];
#pragma unroll
    for (int u = 0; u < J; ++u)
      if (j0 + u < k) {
        const int row = __builtin_amdgcn_readlane(my_row, j0 + u);
        const uint4* src = reinterpret_cast<const uint4*>(Y + (size_t)row * l + CW * lane);
#pragma unroll
        for (int n = 0; n < NC; ++n) v[u][n] = src[n];
      }
#pragma unroll
    for (int u = 0; u < J; ++u)
      if (j0 + u < k) {
        const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j0 + u));
#pragma unroll
        for (int n = 0; n < NC; ++n) {
          const uint32_t w[4] = {v[u][n].x, v[u][n].y, v[u][n].z, v[u][n].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[8 * n + 2 * i] += g * bf16_bits_to_f32(w[i] & 0xFFFFu);
            a[8 * n + 2 * i + 1] += g * bf16_bits_to_f32(w[i] >> 16);
          }
        }
      }
  }
  uint4* dst = reinterpret_cast<uint4*>(y_lat + (size_t)t * l + CW * lane);
#pragma unroll
  for (int n = 0; n < NC; ++n)
    dst[n] = make_uint4(pack_bf16x2(a[8 * n], a[8 * n + 1]), pack_bf16x2(a[8 * n + 2], a[8 * n + 3]),
                        pack_bf16x2(a[8 * n + 4], a[8 * n + 5]), pack_bf16x2(a[8 * n + 6], a[8 * n + 7]));
}

hipError_t launch_combine(const Dims& D, const void* Y, const float* gates, const int32_t* inv, int T, void* y_lat,
                          hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16 && (D.l == 512 || D.l == 1024)) {
    const uint16_t* Yb = static_cast<const uint16_t*>(Y);
    uint16_t* yb = static_cast<uint16_t*>(y_lat);
    if (D.l == 512)
      hipLaunchKernelGGL(k_combine_wide<8>, grid, dim3(256), 0, s, Yb, gates, inv, T, D.k, yb);
    else
      hipLaunchKernelGGL(k_combine_wide<16>, grid, dim3(256), 0, s, Yb, gates, inv, T, D.k, yb);
  } else if (D.bf16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, Y, gates, inv, T, D.l, D.k, y_lat);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, Y, gates, inv, T, D.l, D.k, y_lat);
  return hipGetLastError();
}

// ------------------------------------------------------------ QB update ----
// Largest token count one statistics window may hold: each histogram bin (and
// each sign-rule load) is a 32-bit counter that never exceeds the window's
// token count.  The host refuses an eager call that would pass it
// (MOE_ERR_STATE); replays of a captured graph are not seen by the host, so
// the update kernels check the device's own 64-bit count as well: a window
// past the limit leaves the bias unchanged, writes NaN to every q_e (QB) and
// is cleared.
constexpr unsigned long long kMaxWindowTokens = 0xFFFFFFFFull;

// Per expert (one block each, one thread per bin): read the bin and clear
// it; with A_j = tokens above bin j (a suffix sum: wave shuffles, then the
// wave totals), the one bin with A_j*E < N*k <= (A_j + c_j)*E (exact integer
// tests) holds the score the expert must beat to receive N*k/E tokens; inside
// it the estimate is linear in the bin, as a fraction of the histogram range
// [lo, hi]: u = (j+1)/B - ((N*k - A_j*E) / (E*c_j)) / B and q = lo + (hi - lo)
// * u, fp64 (q = u on [0, 1]).  A window past kMaxWindowTokens marks q NaN.
__global__ __launch_bounds__(256) void k_qb_quantile(uint32_t* __restrict__ hist,
                                                     const unsigned long long* __restrict__ count, int E, int B,
                                                     int k, double lo, double width, double* __restrict__ q) {
#pragma clang fp contract(off)
  __shared__ unsigned long long wtot[4];
  const unsigned long long N = *count;
  if (N == 0) return;
  const int e = blockIdx.x, j = threadIdx.x, lane = j & 63, w = j >> 6;
  unsigned long long c = 0;
  if (j < B) {
    c = hist[(size_t)e * B + j];
    hist[(size_t)e * B + j] = 0u;
  }
  if (N > kMaxWindowTokens) {  // block-uniform
    if (j == 0) q[e] = __builtin_nan("");
    return;
  }
  unsigned long long incl = c;  // inclusive suffix sum inside the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long u = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += u;
  }
  if (lane == 0) wtot[w] = incl;
  __syncthreads();
  for (int w2 = w + 1; w2 < 4; ++w2) incl += wtot[w2];
  if (j < B) {
    const unsigned long long above = incl - c;
    const unsigned long long target = N * (unsigned long long)k, EE = (unsigned long long)E;
    if (above * EE < target && target <= incl * EE) {
      const double frac = (double)(target - above * EE) / (double)(EE * c);
      q[e] = lo + width * ((double)(j + 1) / (double)B - frac / (double)B);
    }
  }
}

// b_e = fp32(mu - q_e), mu the fp64 mean of q summed in expert order (the q
// are staged in LDS by all threads, the sum is one thread's); then the token
// count is cleared.  Keeps the bias when no token was accumulated, or when
// the window passed kMaxWindowTokens (then only the count is cleared).
__global__ __launch_bounds__(1024) void k_qb_bias(const double* __restrict__ q, unsigned long long* __restrict__ count,
                                                  int E, float* __restrict__ bias) {
#pragma clang fp contract(off)
  __shared__ double qs[1024];
  __shared__ double mu_s;
  const unsigned long long N = *count;
  if (N == 0) return;
  if (N > kMaxWindowTokens) {
    __syncthreads();  // every thread has read the count before it is cleared
    if (threadIdx.x == 0) *count = 0ull;
    return;
  }
  for (int e = threadIdx.x; e < E; e += 1024) qs[e] = q[e];
  __syncthreads();
  if (threadIdx.x == 0) {
    double mu = 0.0;
    for (int e = 0; e < E; ++e) mu += qs[e];
    mu_s = mu / (double)E;
  }
  __syncthreads();
  const double mu = mu_s;
  for (int e = threadIdx.x; e < E; e += 1024) bias[e] = (float)(mu - qs[e]);
  __syncthreads();
  if (threadIdx.x == 0) *count = 0ull;
}

hipError_t launch_qb_update(const Dims& D, uint32_t* hist, unsigned long long* count, double* q, float* bias,
                            hipStream_t s) {
  const double lo = (double)D.qb_lo, width = (double)D.qb_hi - (double)D.qb_lo;
  hipLaunchKernelGGL(k_qb_quantile, dim3(D.E), dim3(256), 0, s, hist, count, D.E, D.B, D.k, lo, width, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_qb_bias, dim3(1), dim3(1024), 0, s, q, count, D.E, bias);
  return hipGetLastError();
}

// ------------------------------------------------------- sign-rule bias ----
// Sign-rule balancer (capsule 16 of the "Pretraining a Mini Kimi K3" review):
// b_e += gamma * sign(mean load - n_e).  With S = sum of the loads, the sign
// of S / E - n_e is that of S - E * n_e, compared exactly in 64-bit integers;
// the bias moves by one fp32 add or subtract of gamma (or not at all).  One
// block; the loads and the token count are cleared for the next window.
__global__ __launch_bounds__(1024) void k_sign_bias(uint32_t* __restrict__ load, unsigned long long* __restrict__ count,
                                                    int E, float gamma, float* __restrict__ bias) {
  __shared__ unsigned long long part[16];
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  if (*count > kMaxWindowTokens) {  // loads may have wrapped: keep the bias, clear the window
    __syncthreads();
    if (i < E) load[i] = 0u;
    if (i == 0) *count = 0ull;
    return;
  }
  const uint32_t n = i < E ? load[i] : 0u;
  unsigned long long v = n;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) part[w] = v;
  __syncthreads();
  unsigned long long S = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) S += part[j];
  if (i < E) {
    const long long diff = (long long)S - (long long)E * (long long)n;
    const float b = bias[i];
    bias[i] = diff > 0 ? b + gamma : (diff < 0 ? b - gamma : b);
    load[i] = 0u;
  }
  if (i == 0) *count = 0ull;
}

hipError_t launch_sign_bias(const Dims& D, uint32_t* load, unsigned long long* count, float gamma, float* bias,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_sign_bias, dim3(1), dim3(1024), 0, s, load, count, D.E, gamma, bias);
  return hipGetLastError();
}

// ----------------------------------------------------------------- fill ----
// Zero a 16-byte-aligned region whose size is a multiple of 16 (a kernel
// rather than a memset node, so that the call is safe under graph capture).
// Largest |fast_sigmoid - router_sigmoid| over every fp32 bit pattern,
// kept as the bits of a non-negative float (their integer order is the
// float order), so the maximum does not depend on the order of the blocks.
__global__ __launch_bounds__(256) void k_fast_score_error(uint32_t* __restrict__ out) {
  uint32_t m = 0;
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  for (uint64_t u = (uint64_t)blockIdx.x * 256u + threadIdx.x; u < (1ull << 32); u += stride) {
    const float l = __uint_as_float((uint32_t)u);
    m = max(m, __float_as_uint(fabsf(fast_sigmoid(l) - router_sigmoid(l))));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) atomicMax(out, m);
}

__global__ void k_set_u32(uint32_t* __restrict__ p, uint32_t v) { *p = v; }

hipError_t launch_fast_score_error(float* out, hipStream_t s) {
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, s, o, 0u);
  hipLaunchKernelGGL(k_fast_score_error, dim3(8192), dim3(256), 0, s, o);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace moe
