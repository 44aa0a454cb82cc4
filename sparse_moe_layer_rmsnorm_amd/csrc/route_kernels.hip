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

namespace moe {

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

template <bool BF16>
MOE_DEV uint4 chunk_scale(const uint4& v, float rstd, const float* g) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  if (BF16) {
    const float4 g0 = *reinterpret_cast<const float4*>(g), g1 = *reinterpret_cast<const float4*>(g + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(bf16_bits_to_f32(w[i] & 0xFFFFu) * rstd * gg[2 * i],
                         bf16_bits_to_f32(w[i] >> 16) * rstd * gg[2 * i + 1]);
  } else {
    const float4 g0 = *reinterpret_cast<const float4*>(g);
    const float gg[4] = {g0.x, g0.y, g0.z, g0.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(__uint_as_float(w[i]) * rstd * gg[i]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <bool BF16, int CPL>
__global__ __launch_bounds__(256) void k_rmsnorm(const void* __restrict__ x, const float* __restrict__ gamma,
                                                 void* __restrict__ h, int T, int d, float eps) {
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
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i] = lane + 64 * i < nch ? xr[lane + 64 * i] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < CPL; ++i) ss += chunk_sumsq<BF16>(v[i]);
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) hr[c] = chunk_scale<BF16>(v[i], rstd, gamma + c * EPC);
    }
  } else {
    for (int c = lane; c < nch; c += 64) ss += chunk_sumsq<BF16>(xr[c]);
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < nch; c += 64) hr[c] = chunk_scale<BF16>(xr[c], rstd, gamma + c * EPC);
  }
}

template <bool BF16>
static void rmsnorm_dispatch(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s) {
  const int per_lane = (D.d / (BF16 ? 8 : 4) + 63) / 64;
  dim3 grid((T + 3) / 4), block(256);
  if (per_lane <= 1) hipLaunchKernelGGL((k_rmsnorm<BF16, 1>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps);
  else if (per_lane <= 2) hipLaunchKernelGGL((k_rmsnorm<BF16, 2>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps);
  else if (per_lane <= 4) hipLaunchKernelGGL((k_rmsnorm<BF16, 4>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps);
  else if (per_lane <= 8) hipLaunchKernelGGL((k_rmsnorm<BF16, 8>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps);
  else hipLaunchKernelGGL((k_rmsnorm<BF16, 0>), grid, block, 0, s, x, gamma, h, T, D.d, D.eps);
}

hipError_t launch_rmsnorm(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s) {
  if (D.bf16)
    rmsnorm_dispatch<true>(D, x, gamma, h, T, s);
  else
    rmsnorm_dispatch<false>(D, x, gamma, h, T, s);
  return hipGetLastError();
}

// -------------------------------------------------- scores + top-k ----
// One block per chunk of kChunk = 32 tokens, kTopkNT tokens per wavefront
// ranked side by side (independent chains hide each other's latency).  Lane i holds experts i, i+64, ... .  Each of the k rounds takes
// the wave-wide maximum (DPP, no LDS) of the order key of v = s + b; among
// equal keys the lowest expert index wins (first the lowest column c of any
// lane holding the key, then the lowest such lane, by ballots).  Gates are
// the chosen unbiased scores over their fp32 sum in slot order.  The chunk's
// selections leave as one 32-bit token mask per expert: bitmap[chunk][e] bit
// t%32 is set iff token t picked e.
template <int CPL, int NT>
MOE_DEV void topk_tokens(const float* __restrict__ logits, const float (&b)[CPL], const int (&t)[NT], int E, int k,
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
        key[n][c] = float_order_key(s[n][c] + b[c]);  // > 0 for any finite v
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

#ifndef MOE_TOPK_NT
#define MOE_TOPK_NT 2
#endif
constexpr int kTopkNT = MOE_TOPK_NT;                    // tokens ranked side by side per wavefront
constexpr int kTopkThreads = kChunk / kTopkNT * 64;      // one token group per wavefront

template <int CPL>
MOE_DEV void topk_block(int chunk, uint32_t* mask, const float* __restrict__ logits, const float* __restrict__ bias,
                        int T, int E, int k, float scale, int32_t* __restrict__ idx, float* __restrict__ gates,
                        uint32_t* __restrict__ bitmap) {
  constexpr int NW = kChunk / kTopkNT;
  for (int i = threadIdx.x; i < E; i += kTopkThreads) mask[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float b[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    b[c] = e < E ? bias[e] : 0.f;
  }
  int t[kTopkNT];
  int n = 0;
#pragma unroll
  for (int u = 0; u < kTopkNT; ++u) {
    t[u] = chunk * kChunk + wave + NW * u;
    n += t[u] < T;
  }
  if (n == kTopkNT) {
    topk_tokens<CPL, kTopkNT>(logits, b, t, E, k, scale, idx, gates, mask);
  } else {
    for (int u = 0; u < n; ++u) {  // ragged last chunk: one at a time
      const int t1[1] = {t[u]};
      topk_tokens<CPL, 1>(logits, b, t1, E, k, scale, idx, gates, mask);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kTopkThreads) bitmap[(size_t)chunk * E + i] = mask[i];
}

// ---------------------------------------------------------- QB histogram ----
// The state keeps the histogram as kHistSlices token slices [slice][E][B].
// Block (16-expert group, slice) counts its tokens' score bins in LDS with
// integer atomics (order-free) and adds them to its own rows of its own slice
// (no other block of the launch writes them), so no reduction pass is needed
// per forward; qb_update sums the slices.
MOE_DEV void hist_block(int group, int ts, uint32_t* lh, const float* __restrict__ logits, int T, int E, int B,
                        int tps, uint32_t* __restrict__ hist, unsigned long long* __restrict__ count) {
  constexpr int TR = kTopkThreads / kHistExperts;  // token rows in flight per step
  const int e0 = group * kHistExperts;
  const int ne = min(kHistExperts, E - e0);
  const int nb = kHistExperts * B;
  for (int i = threadIdx.x; i < nb; i += kTopkThreads) lh[i] = 0;
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
      atomicAdd(&row[score_bin(router_sigmoid(l0), B)], 1u);
      atomicAdd(&row[score_bin(router_sigmoid(l1), B)], 1u);
    }
    for (; t < te; t += TR) atomicAdd(&row[score_bin(router_sigmoid(logits[(size_t)t * E + e]), B)], 1u);
  }
  __syncthreads();
  if (tb < T) {
    uint32_t* dst = hist + ((size_t)ts * E + e0) * B;
    for (int i = threadIdx.x; i < ne * B; i += kTopkThreads) {
      const uint32_t v = lh[i];
      if (v) dst[i] += v;
    }
  }
  if (group == 0 && ts == 0 && threadIdx.x == 0) *count += (unsigned long long)T;
}

// One launch for the scores: blocks [0, nchunks) rank the chunks; in
// training mode blocks past them build the QB histogram from the same
// logits (independent work side by side instead of two launches).
template <int CPL>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ logits,
                                                       const float* __restrict__ bias, int T, int E, int k,
                                                       float scale, int32_t* __restrict__ idx,
                                                       float* __restrict__ gates, uint32_t* __restrict__ bitmap,
                                                       int nchunks, int B, int tps, uint32_t* __restrict__ hist,
                                                       unsigned long long* __restrict__ count) {
  __shared__ uint32_t smem[kHistExperts * 256];
  static_assert(kHistExperts * 256 >= 1024, "the top-k masks fit");
  if ((int)blockIdx.x < nchunks) {
    topk_block<CPL>(blockIdx.x, smem, logits, bias, T, E, k, scale, idx, gates, bitmap);
  } else {
    const int hb = blockIdx.x - nchunks, groups = (E + kHistExperts - 1) / kHistExperts;
    hist_block(hb % groups, hb / groups, smem, logits, T, E, B, tps, hist, count);
  }
}

hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       uint32_t* bitmap, uint32_t* hist, unsigned long long* count, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cpl = (D.E + 63) / 64;
  const int tps = (T + kHistSlices - 1) / kHistSlices;
  const int hblocks = hist ? (D.E + kHistExperts - 1) / kHistExperts * kHistSlices : 0;
  dim3 grid(nchunks + hblocks), block(kTopkThreads);
#define MOE_TOPK(C)                                                                                                 \
  hipLaunchKernelGGL(k_topk<C>, grid, block, 0, s, logits, bias, T, D.E, D.k, D.routed_scale, idx, gates, bitmap, \
                     nchunks, D.B, tps, hist, count)
  if (cpl <= 1) MOE_TOPK(1);
  else if (cpl <= 2) MOE_TOPK(2);
  else if (cpl <= 4) MOE_TOPK(4);
  else if (cpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

// ------------------------------------------------------- counts / scan ----
// Two-level exclusive prefix sums of the per-(chunk, expert) selection counts
// popcount(bitmap[c][e]).  Local: per super-chunk of kSuper chunks, one lane
// per expert walks its chunks: cbase[c][e] = count of expert e in the earlier
// chunks of the super-chunk; sbase[sc][e] = the super-chunk's total.
__global__ __launch_bounds__(256) void k_scan_local(const uint32_t* __restrict__ bitmap, int nchunks, int E,
                                                    int32_t* __restrict__ cbase, int32_t* __restrict__ sbase) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int sc = blockIdx.y * 4 + wave;
  const int c0 = sc * kSuper;
  if (e >= E || c0 >= nchunks) return;
  uint32_t m[kSuper];  // all loads of the super-chunk in flight together
#pragma unroll
  for (int j = 0; j < kSuper; ++j) m[j] = c0 + j < nchunks ? bitmap[(size_t)(c0 + j) * E + e] : 0u;
  int run = 0;
#pragma unroll
  for (int j = 0; j < kSuper; ++j) {
    if (c0 + j < nchunks) cbase[(size_t)(c0 + j) * E + e] = run;
    run += __popc(m[j]);
  }
  sbase[(size_t)sc * E + e] = run;
}

// Global (one block of 1024 threads, one expert per thread): per expert, the
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
  // per expert (E <= 1024): first row, count, inclusive tile prefixes of both tables
  __shared__ int s_row0[1024], s_cnt[1024], s_t[1024], s_u[1024];
  constexpr int kReg = 16;  // up to this many super-chunk totals stay in registers
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  // at most 8 tiles of kExpertBM rows per expert on average: one thread per
  // expert writes its tiles (cheaper than a block-wide pass at these sizes)
  const bool few = (long long)T * k <= 8LL * kExpertBM * E;
  int c = 0;
  int v[kReg];
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
    } else {
#pragma unroll 16
      for (int sc = 0; sc < nsuper; ++sc) {
        const size_t j = (size_t)sc * E + i;
        const int x = sbase[j];
        sbase[j] = run;
        run += x;
      }
    }
    s_row0[i] = r - c;
    s_cnt[i] = c;
    s_t[i] = t;
    s_u[i] = u;
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
  if (few) return;
  __syncthreads();
  // Many tiles per expert: the tile tables are spread over the whole block;
  // tile g belongs to the expert whose tile range holds it (binary search
  // over the inclusive prefixes).
  auto fill = [&](const int* pre, int bm, int2* info) {
    const int total = pre[E - 1];
    for (int g = i; g < total; g += 1024) {
      int lo = 0, hi = E - 1;  // first e with pre[e] > g
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] > g) hi = mid;
        else lo = mid + 1;
      }
      const int j = g - (lo > 0 ? pre[lo - 1] : 0);
      info[g] = make_int2(s_row0[lo] + j * bm, (lo << 8) | min(bm, s_cnt[lo] - j * bm));
    }
  };
  fill(s_t, kExpertBM, tile_info);
  if (tile_info2) fill(s_u, kExpertBM2, tile_info2);
}

hipError_t launch_scan(const Dims& D, const uint32_t* bitmap, int T, int32_t* cbase, int32_t* sbase, int32_t* counts,
                       int32_t* offsets, int32_t* tile_offsets, int2* tile_info, uint32_t* load,
                       unsigned long long* count, hipStream_t s, int32_t* tile_offsets2, int2* tile_info2) {
  if ((tile_offsets2 == nullptr) != (tile_info2 == nullptr)) return hipErrorInvalidValue;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int nsuper = (nchunks + kSuper - 1) / kSuper;
  dim3 g1((D.E + 63) / 64, (nsuper + 3) / 4);
  hipLaunchKernelGGL(k_scan_local, g1, dim3(256), 0, s, bitmap, nchunks, D.E, cbase, sbase);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_global, dim3(1), dim3(1024), 0, s, sbase, nsuper, D.E, counts, offsets, tile_offsets,
                     tile_info, load, load ? count : nullptr, T, D.k, tile_offsets2, tile_info2);
  return hipGetLastError();
}

// -------------------------------------------------------------- scatter ----
// Stable rows without order-dependent atomics, one thread per (t, j): the row
// of (t, j) in expert e's group is the super-chunk base + the chunk base +
// the number of earlier tokens of the chunk in the chunk's mask for e.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, const uint32_t* __restrict__ bitmap,
                                                 const int32_t* __restrict__ cbase, const int32_t* __restrict__ sbase,
                                                 int T, int E, int k, int32_t* __restrict__ perm_src,
                                                 int32_t* __restrict__ inv, const uint32_t* __restrict__ zs,
                                                 uint32_t* __restrict__ Xs, int s4) {
  const int Tk = T * k;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= Tk) return;
  const int t = p / k;
  const int e = idx[p];
  const int c = t / kChunk;
  const size_t ce = (size_t)c * E + e;
  const uint32_t below = bitmap[ce] & ((1u << (t % kChunk)) - 1u);
  const int row = sbase[(size_t)(c / kSuper) * E + e] + cbase[ce] + __popc(below);
  inv[p] = row;
  if ((unsigned)row < (unsigned)Tk) {  // always true for a consistent permutation
    perm_src[row] = t;
    for (int q = 0; q < s4; ++q) Xs[(size_t)row * s4 + q] = zs[(size_t)t * s4 + q];
  }
}

hipError_t launch_scatter(const Dims& D, const int32_t* idx, const uint32_t* bitmap, const int32_t* cbase,
                          const int32_t* sbase, int T, int32_t* perm_src, int32_t* inv, hipStream_t s,
                          const uint8_t* zs, uint8_t* Xs, int s_ld) {
  const long long Tk = (long long)T * D.k;
  if (zs && s_ld % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)((Tk + 255) / 256)), dim3(256), 0, s, idx, bitmap, cbase, sbase, T,
                     D.E, D.k, perm_src, inv, reinterpret_cast<const uint32_t*>(zs), reinterpret_cast<uint32_t*>(Xs),
                     zs ? s_ld / 4 : 0);
  return hipGetLastError();
}

// -------------------------------------------------------------- combine ----
// y_lat[t] = sum_j g[t,j] Y[inv[t,j]] in slot order, fp32, stored in the
// activation dtype.  One wavefront per token; lane c handles 4 latent
// columns per 4*64-column stripe.
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
  for (int q = lane; q < nq; q += 64) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < k; ++j) {
      // readlane, not a shuffle: lanes past l/4 are inactive in this loop
      const int row = __builtin_amdgcn_readlane(my_row, j);
      const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j));
      if (BF16) {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(Y) + (size_t)row * l + 4 * q);
        a0 += g * bf16_bits_to_f32(v.x & 0xFFFFu);
        a1 += g * bf16_bits_to_f32(v.x >> 16);
        a2 += g * bf16_bits_to_f32(v.y & 0xFFFFu);
        a3 += g * bf16_bits_to_f32(v.y >> 16);
      } else {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(Y) + (size_t)row * l + 4 * q);
        a0 += g * v.x;
        a1 += g * v.y;
        a2 += g * v.z;
        a3 += g * v.w;
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

hipError_t launch_combine(const Dims& D, const void* Y, const float* gates, const int32_t* inv, int T, void* y_lat,
                          hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, s, Y, gates, inv, T, D.l, D.k, y_lat);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, s, Y, gates, inv, T, D.l, D.k, y_lat);
  return hipGetLastError();
}

// ------------------------------------------------------------ QB update ----
// Per expert (one block each, one thread per bin): sum the bin over the
// histogram slices and clear it; with A_j = tokens above bin j (a suffix sum:
// wave shuffles, then the wave totals), the one bin with
// A_j*E < N*k <= (A_j + c_j)*E (exact integer tests) holds the score the
// expert must beat to receive N*k/E tokens; inside it the estimate is linear:
// q = (j+1)/B - ((N*k - A_j*E) / (E*c_j)) / B, fp64.
__global__ __launch_bounds__(256) void k_qb_quantile(uint32_t* __restrict__ hist,
                                                     const unsigned long long* __restrict__ count, int E, int B,
                                                     int k, double* __restrict__ q) {
#pragma clang fp contract(off)
  __shared__ unsigned long long wtot[4];
  const unsigned long long N = *count;
  if (N == 0) return;
  const int e = blockIdx.x, j = threadIdx.x, lane = j & 63, w = j >> 6;
  unsigned long long c = 0;
  if (j < B) {
    uint32_t v[kHistSlices];
#pragma unroll
    for (int sl = 0; sl < kHistSlices; ++sl) v[sl] = hist[((size_t)sl * E + e) * B + j];
#pragma unroll
    for (int sl = 0; sl < kHistSlices; ++sl) {
      c += v[sl];
      hist[((size_t)sl * E + e) * B + j] = 0u;
    }
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
      q[e] = (double)(j + 1) / (double)B - frac / (double)B;
    }
  }
}

// b_e = fp32(mu - q_e), mu the fp64 mean of q summed in expert order (the q
// are staged in LDS by all threads, the sum is one thread's); then the token
// count is cleared.  Keeps the bias when no token was accumulated.
__global__ __launch_bounds__(1024) void k_qb_bias(const double* __restrict__ q, unsigned long long* __restrict__ count,
                                                  int E, float* __restrict__ bias) {
#pragma clang fp contract(off)
  __shared__ double qs[1024];
  __shared__ double mu_s;
  if (*count == 0) return;
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

hipError_t launch_qb_quantile(const Dims& D, uint32_t* hist, const unsigned long long* count, double* q,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_qb_quantile, dim3(D.E), dim3(256), 0, s, hist, count, D.E, D.B, D.k, q);
  return hipGetLastError();
}

hipError_t launch_qb_bias(const Dims& D, const double* q, unsigned long long* count, float* bias, hipStream_t s) {
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
