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
// + eps), fp32 arithmetic, stored in the activation dtype.
template <bool BF16>
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
  for (int c = lane; c < nch; c += 64) {
    uint4 v = xr[c];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (BF16) {
        float a = bf16_bits_to_f32(w[i] & 0xFFFFu), b = bf16_bits_to_f32(w[i] >> 16);
        ss += a * a + b * b;
      } else {
        float a = __uint_as_float(w[i]);
        ss += a * a;
      }
    }
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < nch; c += 64) {
    uint4 v = xr[c];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const float* g = gamma + c * EPC;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (BF16) {
        float a = bf16_bits_to_f32(w[i] & 0xFFFFu) * rstd * g[2 * i];
        float b = bf16_bits_to_f32(w[i] >> 16) * rstd * g[2 * i + 1];
        o[i] = pack_bf16x2(a, b);
      } else {
        o[i] = __float_as_uint(__uint_as_float(w[i]) * rstd * g[i]);
      }
    }
    hr[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_rmsnorm(const Dims& D, const void* x, const float* gamma, void* h, int T, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16)
    hipLaunchKernelGGL(k_rmsnorm<true>, grid, dim3(256), 0, s, x, gamma, h, T, D.d, D.eps);
  else
    hipLaunchKernelGGL(k_rmsnorm<false>, grid, dim3(256), 0, s, x, gamma, h, T, D.d, D.eps);
  return hipGetLastError();
}

// -------------------------------------------------- scores + top-k ----
// One block per chunk of kChunk = 32 tokens, 8 wavefronts, one token per
// wavefront at a time (the next token's logits are loaded while the current
// one is ranked).  Lane i holds experts i, i+64, ... .  Each of the k rounds
// takes the wave-wide maximum (DPP, no LDS) of the 64-bit key (order key of
// v = s + b, then the complement of the expert index), so equal v go to the
// lower index.  Gates are the chosen unbiased scores over their fp32 sum in
// slot order.  The chunk's selections leave as one 32-bit token mask per
// expert: bitmap[chunk][e] bit t%32 is set iff token t picked e.
template <int CPL>
__global__ __launch_bounds__(512) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int k, float scale, int32_t* __restrict__ idx,
                                              float* __restrict__ gates, uint32_t* __restrict__ bitmap) {
#pragma clang fp contract(off)
  __shared__ uint32_t mask[1024];
  for (int i = threadIdx.x; i < E; i += 512) mask[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float b[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    b[c] = e < E ? bias[e] : 0.f;
  }
  float nxt[CPL];
  auto load = [&](int t) {
    const float* lr = logits + (size_t)t * E;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      nxt[c] = e < E ? lr[e] : 0.f;
    }
  };
  int t = blockIdx.x * kChunk + wave;
  if (t < T) load(t);
  for (int it = 0; it < kChunk / 8; ++it, t += 8) {
    if (t >= T) break;  // uniform across the wavefront
    float s[CPL];
    unsigned long long key[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) s[c] = nxt[c];
    if (it + 1 < kChunk / 8 && t + 8 < T) load(t + 8);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      if (e < E) {
        s[c] = router_sigmoid(s[c]);
        const float v = s[c] + b[c];
        key[c] = ((unsigned long long)float_order_key(v) << 32) | (0xFFFFFFFFu - (uint32_t)e);
      } else {
        s[c] = 0.f;
        key[c] = 0ull;
      }
    }
    float S = 0.f, my_s = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      unsigned long long best = key[0];
#pragma unroll
      for (int c = 1; c < CPL; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const int owner = e & 63, oc = e >> 6;
      float sv = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (c == oc) {
          sv = s[c];
          if (lane == owner) key[c] = 0ull;
        }
      }
      const float se = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), owner));
      S = (j == 0) ? se : S + se;
      if (lane == j) {
        my_s = se;
        my_e = e;
      }
    }
    if (lane < k) {
      const float g = (my_s / S) * scale;
      idx[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = g;
      atomicOr(&mask[my_e], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 512) bitmap[(size_t)blockIdx.x * E + i] = mask[i];
}

hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       uint32_t* bitmap, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cpl = (D.E + 63) / 64;
  dim3 grid(nchunks), block(512);
#define MOE_TOPK(C) \
  hipLaunchKernelGGL(k_topk<C>, grid, block, 0, s, logits, bias, T, D.E, D.k, D.routed_scale, idx, gates, bitmap)
  if (cpl <= 1) MOE_TOPK(1);
  else if (cpl <= 2) MOE_TOPK(2);
  else if (cpl <= 4) MOE_TOPK(4);
  else if (cpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

// ---------------------------------------------------------- QB histogram ----
// The state keeps the histogram as kHistSlices token slices [slice][E][B].
// Block (64-expert group, slice) counts its tokens' score bins in LDS with
// integer atomics (order-free) and adds them to its own rows of its own slice
// (no other block of the launch writes them), so no reduction pass is needed
// per forward; qb_update sums the slices.
__global__ __launch_bounds__(1024) void k_hist(const float* __restrict__ logits, int T, int E, int B, int tps,
                                               uint32_t* __restrict__ hist, unsigned long long* __restrict__ count) {
  __shared__ uint32_t lh[kHistExperts * 256];
  const int e0 = blockIdx.x * kHistExperts, ts = blockIdx.y;
  const int ne = min(kHistExperts, E - e0);
  const int nb = kHistExperts * B;
  for (int i = threadIdx.x; i < nb; i += 1024) lh[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = e0 + lane;
  const int tb = ts * tps, te = min(T, tb + tps);
  if (e < E) {
    int t = tb + wave;
    for (; t + 48 < te; t += 64) {
      const float l0 = logits[(size_t)t * E + e], l1 = logits[(size_t)(t + 16) * E + e];
      const float l2 = logits[(size_t)(t + 32) * E + e], l3 = logits[(size_t)(t + 48) * E + e];
      atomicAdd(&lh[lane * B + score_bin(router_sigmoid(l0), B)], 1u);
      atomicAdd(&lh[lane * B + score_bin(router_sigmoid(l1), B)], 1u);
      atomicAdd(&lh[lane * B + score_bin(router_sigmoid(l2), B)], 1u);
      atomicAdd(&lh[lane * B + score_bin(router_sigmoid(l3), B)], 1u);
    }
    for (; t < te; t += 16) atomicAdd(&lh[lane * B + score_bin(router_sigmoid(logits[(size_t)t * E + e]), B)], 1u);
  }
  __syncthreads();
  if (tb < T) {
    uint32_t* dst = hist + ((size_t)ts * E + e0) * B;
    for (int i = threadIdx.x; i < ne * B; i += 1024) {
      const uint32_t v = lh[i];
      if (v) dst[i] += v;
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *count += (unsigned long long)T;
}

hipError_t launch_hist(const Dims& D, const float* logits, int T, uint32_t* hist, unsigned long long* count,
                       hipStream_t s) {
  const int tps = (T + kHistSlices - 1) / kHistSlices;
  dim3 grid((D.E + kHistExperts - 1) / kHistExperts, kHistSlices);
  hipLaunchKernelGGL(k_hist, grid, dim3(1024), 0, s, logits, T, D.E, D.B, tps, hist, count);
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
  const int c1 = min(nchunks, c0 + kSuper);
  int run = 0;
  for (int c = c0; c < c1; ++c) {
    const size_t i = (size_t)c * E + e;
    const int v = __popc(bitmap[i]);
    cbase[i] = run;
    run += v;
  }
  sbase[(size_t)sc * E + e] = run;
}

// Global (one block of 1024 threads): per expert, the total and the exclusive
// prefix over super-chunks (sbase becomes the absolute first row of each
// super-chunk's part of the expert's group); over experts, the row offsets
// and the first m-tile of each expert for the grouped GEMMs (tiles of
// kExpertBM rows; an empty expert has none).
__global__ __launch_bounds__(1024) void k_scan_global(int32_t* __restrict__ sbase, int nsuper, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ tile_offsets, int2* __restrict__ tile_info) {
  __shared__ int wsum_r[16], wsum_t[16];
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  int c = 0;
  if (i < E) {
#pragma unroll 8
    for (int sc = 0; sc < nsuper; ++sc) c += sbase[(size_t)sc * E + i];
  }
  const int tl = (c + kExpertBM - 1) / kExpertBM;
  int r = c, t = tl;  // inclusive wave scans
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ro = __shfl_up(r, o, 64), to = __shfl_up(t, o, 64);
    if (lane >= o) {
      r += ro;
      t += to;
    }
  }
  if (lane == 63) {
    wsum_r[w] = r;
    wsum_t[w] = t;
  }
  __syncthreads();
  int br = 0, bt = 0;
  for (int j = 0; j < w; ++j) {
    br += wsum_r[j];
    bt += wsum_t[j];
  }
  r += br;
  t += bt;
  if (i < E) {
    counts[i] = c;
    offsets[i + 1] = r;
    tile_offsets[i + 1] = t;
    int run = r - c;  // exclusive offset of expert i
    for (int sc = 0; sc < nsuper; ++sc) {
      const size_t j = (size_t)sc * E + i;
      const int v = sbase[j];
      sbase[j] = run;
      run += v;
    }
    const int row0 = r - c, tile0 = t - tl;
    for (int j = 0; j < tl; ++j)
      tile_info[tile0 + j] = make_int2(row0 + j * kExpertBM, (i << 8) | min(kExpertBM, c - j * kExpertBM));
  }
  if (i == 0) {
    offsets[0] = 0;
    tile_offsets[0] = 0;
  }
}

hipError_t launch_scan(const Dims& D, const uint32_t* bitmap, int T, int32_t* cbase, int32_t* sbase, int32_t* counts,
                       int32_t* offsets, int32_t* tile_offsets, int2* tile_info, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int nsuper = (nchunks + kSuper - 1) / kSuper;
  dim3 g1((D.E + 63) / 64, (nsuper + 3) / 4);
  hipLaunchKernelGGL(k_scan_local, g1, dim3(256), 0, s, bitmap, nchunks, D.E, cbase, sbase);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_global, dim3(1), dim3(1024), 0, s, sbase, nsuper, D.E, counts, offsets, tile_offsets,
                     tile_info);
  return hipGetLastError();
}

// -------------------------------------------------------------- scatter ----
// Stable rows without order-dependent atomics.  One wavefront per token:
// lane j < k finds the row of (t, j) in expert e's group as the super-chunk
// base + the chunk base + the number of earlier tokens of the chunk in the
// chunk's mask for e; then the wavefront copies the token's latent row z[t]
// to the dispatch buffer X at each of its k rows (coalesced 16-byte pieces).
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, const uint32_t* __restrict__ bitmap,
                                                 const int32_t* __restrict__ cbase, const int32_t* __restrict__ sbase,
                                                 const uint4* __restrict__ z, int T, int E, int k, int row16,
                                                 int32_t* __restrict__ perm_src, int32_t* __restrict__ inv,
                                                 uint4* __restrict__ X) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int Tk = T * k;
  int my_row = -1;
  if (lane < k) {
    const int e = idx[(size_t)t * k + lane];
    const int c = t / kChunk;
    const size_t ce = (size_t)c * E + e;
    const uint32_t below = bitmap[ce] & ((1u << (t % kChunk)) - 1u);
    const int row = sbase[(size_t)(c / kSuper) * E + e] + cbase[ce] + __popc(below);
    inv[(size_t)t * k + lane] = row;
    if ((unsigned)row < (unsigned)Tk) {  // always true for a consistent permutation
      perm_src[row] = t;
      my_row = row;
    }
  }
  const uint4* src = z + (size_t)t * row16;
  for (int c = lane; c < row16; c += 64) {
    const uint4 v = src[c];
    for (int j = 0; j < k; ++j) {
      const int row = __builtin_amdgcn_readlane(my_row, j);
      if (row >= 0) X[(size_t)row * row16 + c] = v;
    }
  }
}

hipError_t launch_scatter(const Dims& D, const int32_t* idx, const uint32_t* bitmap, const int32_t* cbase,
                          const int32_t* sbase, int T, const void* z, int32_t* perm_src, int32_t* inv, void* X,
                          hipStream_t s) {
  const int row16 = (z && X) ? D.l * (D.bf16 ? 2 : 4) / 16 : 0;  // routing only: no dispatch copy
  hipLaunchKernelGGL(k_scatter, dim3((T + 3) / 4), dim3(256), 0, s, idx, bitmap, cbase, sbase,
                     static_cast<const uint4*>(z), T, D.E, D.k, row16, perm_src, inv, static_cast<uint4*>(X));
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
      const int row = __shfl(my_row, j, 64);
      const float g = __shfl(my_g, j, 64);
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
// histogram slices and clear it; with A_j = tokens above bin j (a parallel
// suffix sum), the one bin with A_j*E < N*k <= (A_j + c_j)*E (exact integer
// tests) holds the score the expert must beat to receive N*k/E tokens; inside
// it the estimate is linear: q = (j+1)/B - ((N*k - A_j*E) / (E*c_j)) / B, fp64.
__global__ __launch_bounds__(256) void k_qb_quantile(uint32_t* __restrict__ hist,
                                                     const unsigned long long* __restrict__ count, int E, int B,
                                                     int k, double* __restrict__ q) {
#pragma clang fp contract(off)
  __shared__ unsigned long long suf[2][256];
  const unsigned long long N = *count;
  if (N == 0) return;
  const int e = blockIdx.x, j = threadIdx.x;
  unsigned long long c = 0;
  if (j < B) {
#pragma unroll 4
    for (int sl = 0; sl < kHistSlices; ++sl) {
      uint32_t* p = hist + ((size_t)sl * E + e) * B + j;
      c += *p;
      *p = 0u;
    }
  }
  // inclusive suffix sums over bins (Hillis-Steele, double-buffered)
  int cur = 0;
  suf[0][j] = c;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const unsigned long long v = suf[cur][j] + (j + o < 256 ? suf[cur][j + o] : 0ull);
    suf[cur ^ 1][j] = v;
    cur ^= 1;
    __syncthreads();
  }
  if (j == 0) q[e] = 0.0;
  __syncthreads();
  if (j < B) {
    const unsigned long long incl = suf[cur][j], above = incl - c;
    const unsigned long long target = N * (unsigned long long)k, EE = (unsigned long long)E;
    if (above * EE < target && target <= incl * EE) {
      const double frac = (double)(target - above * EE) / (double)(EE * c);
      q[e] = (double)(j + 1) / (double)B - frac / (double)B;
    }
  }
}

// b_e = fp32(mu - q_e), mu the fp64 mean of q summed in expert order; then the
// token count is cleared.  Keeps the bias when no token was accumulated.
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
#pragma unroll 8
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
