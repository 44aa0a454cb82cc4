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
// One block per chunk of 64 tokens, one wavefront per token at a time.  Lane
// i holds experts i, i+64, ... .  Each of the k rounds takes the wave-wide
// maximum of the 64-bit key (order key of v = s + b, then the complement of
// the expert index), so equal v go to the lower index.  Gates are the chosen
// unbiased scores over their fp32 sum in slot order.  The chunk's per-expert
// counts go to chunk_counts[chunk][E] (LDS integer atomics: order-free).
template <int CPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int T, int E, int k, float scale, int32_t* __restrict__ idx,
                                              float* __restrict__ gates, int32_t* __restrict__ chunk_counts) {
#pragma clang fp contract(off)
  __shared__ int cnt[1024];
  for (int i = threadIdx.x; i < E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float b[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    b[c] = e < E ? bias[e] : 0.f;
  }
  const int t0 = blockIdx.x * kChunk;
  for (int tt = wave; tt < kChunk; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* lr = logits + (size_t)t * E;
    float s[CPL];
    unsigned long long key[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      if (e < E) {
        s[c] = router_sigmoid(lr[e]);
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
      unsigned long long best = 0ull;
#pragma unroll
      for (int c = 0; c < CPL; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const int owner = e & 63;
      float se = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (lane == owner && c == (e >> 6)) {
          se = s[c];
          key[c] = 0ull;
        }
      }
      se = __shfl(se, owner, 64);
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
      atomicAdd(&cnt[my_e], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += 256) chunk_counts[(size_t)blockIdx.x * E + i] = cnt[i];
}

hipError_t launch_topk(const Dims& D, const float* logits, const float* bias, int T, int32_t* idx, float* gates,
                       int32_t* chunk_counts, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cpl = (D.E + 63) / 64;
  dim3 grid(nchunks), block(256);
#define MOE_TOPK(C) \
  hipLaunchKernelGGL(k_topk<C>, grid, block, 0, s, logits, bias, T, D.E, D.k, D.routed_scale, idx, gates, chunk_counts)
  if (cpl <= 1) MOE_TOPK(1);
  else if (cpl <= 2) MOE_TOPK(2);
  else if (cpl <= 4) MOE_TOPK(4);
  else if (cpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

// ---------------------------------------------------------- QB histogram ----
// Block (expert slice of 64, token slice): LDS histogram [64][B] with integer
// atomics (order-free), then either written to its own partial slot or, when
// there is only one token slice, added to the state histogram directly (each
// block owns its experts' rows).
int hist_token_slices(int T, int E) {
  const int es = (E + kHistExperts - 1) / kHistExperts;
  int want = (256 + es - 1) / es;               // about one block per CU
  int by_tokens = (T + 255) / 256;              // at least 256 tokens per slice
  int n = want < by_tokens ? want : by_tokens;
  return n < 1 ? 1 : n;
}

__global__ __launch_bounds__(1024) void k_hist(const float* __restrict__ logits, int T, int E, int B, int tps,
                                               uint32_t* __restrict__ partial, uint32_t* __restrict__ hist,
                                               unsigned long long* __restrict__ count) {
  __shared__ uint32_t lh[kHistExperts * 256];
  const int e0 = blockIdx.x * kHistExperts, ts = blockIdx.y;
  const int nb = kHistExperts * B;
  for (int i = threadIdx.x; i < nb; i += 1024) lh[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = e0 + lane;
  const int tb = ts * tps, te = min(T, tb + tps);
  if (e < E) {
    for (int t = tb + wave; t < te; t += 16) {
      const float sc = router_sigmoid(logits[(size_t)t * E + e]);
      atomicAdd(&lh[lane * B + score_bin(sc, B)], 1u);
    }
  }
  __syncthreads();
  const int ne = min(kHistExperts, E - e0);
  if (partial) {
    uint32_t* dst = partial + ((size_t)ts * E + e0) * B;
    for (int i = threadIdx.x; i < ne * B; i += 1024) dst[i] = lh[i];
  } else {
    uint32_t* dst = hist + (size_t)e0 * B;
    for (int i = threadIdx.x; i < ne * B; i += 1024) dst[i] += lh[i];
    if (blockIdx.x == 0 && threadIdx.x == 0) *count += (unsigned long long)T;
  }
}

__global__ __launch_bounds__(256) void k_hist_reduce(const uint32_t* __restrict__ partial, int nslices, int EB,
                                                     int T, uint32_t* __restrict__ hist,
                                                     unsigned long long* __restrict__ count) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < EB) {
    uint32_t acc = hist[i];
    for (int sl = 0; sl < nslices; ++sl) acc += partial[(size_t)sl * EB + i];
    hist[i] = acc;
  }
  if (i == 0) *count += (unsigned long long)T;
}

hipError_t launch_hist(const Dims& D, const float* logits, int T, uint32_t* partial, uint32_t* hist,
                       unsigned long long* count, hipStream_t s) {
  const int ns = hist_token_slices(T, D.E);
  const int tps = (T + ns - 1) / ns;
  dim3 grid((D.E + kHistExperts - 1) / kHistExperts, ns);
  hipLaunchKernelGGL(k_hist, grid, dim3(1024), 0, s, logits, T, D.E, D.B, tps, ns > 1 ? partial : nullptr, hist,
                     count);
  return hipGetLastError();
}

hipError_t launch_hist_reduce(const Dims& D, const uint32_t* partial, int nslices, int T, uint32_t* hist,
                              unsigned long long* count, hipStream_t s) {
  const int EB = D.E * D.B;
  hipLaunchKernelGGL(k_hist_reduce, dim3((EB + 255) / 256), dim3(256), 0, s, partial, nslices, EB, T, hist, count);
  return hipGetLastError();
}

// ------------------------------------------------------- counts / scan ----
// Per expert, exclusive prefix over the chunks of chunk_counts[chunk][E] (in
// place: it becomes each chunk's base row inside the expert's group) and the
// expert's total.  64 experts per block (one per lane, coalesced rows), the
// chunks split over 16 wavefronts.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ cc, int nchunks, int E,
                                               int32_t* __restrict__ counts) {
  __shared__ int part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int per = (nchunks + 15) / 16;
  const int c0 = min(nchunks, w * per), c1 = min(nchunks, c0 + per);
  int sum = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c) sum += cc[(size_t)c * E + e];
  part[w][lane] = sum;
  __syncthreads();
  int base = 0, total = 0;
  for (int i = 0; i < 16; ++i) {
    const int v = part[i][lane];
    base += i < w ? v : 0;
    total += v;
  }
  if (e < E) {
    int run = base;
    for (int c = c0; c < c1; ++c) {
      const int v = cc[(size_t)c * E + e];
      cc[(size_t)c * E + e] = run;
      run += v;
    }
    if (w == 0) counts[e] = total;
  }
}

hipError_t launch_scan(const Dims& D, int32_t* chunk_counts, int nchunks, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3((D.E + 63) / 64), dim3(1024), 0, s, chunk_counts, nchunks, D.E, counts);
  return hipGetLastError();
}

// Exclusive prefix sums over experts: row offsets[E+1] and, for the grouped
// GEMMs, the first m-tile of each expert tile_offsets[E+1] (tiles of
// kExpertBM rows; an empty expert has none).  One block of 1024 threads.
__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts, int E,
                                                  int32_t* __restrict__ offsets, int32_t* __restrict__ tile_offsets) {
  __shared__ int wsum_r[16], wsum_t[16];
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  const int c = i < E ? counts[i] : 0;
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
    offsets[i + 1] = r;
    tile_offsets[i + 1] = t;
  }
  if (i == 0) {
    offsets[0] = 0;
    tile_offsets[0] = 0;
  }
}

hipError_t launch_offsets(const Dims& D, const int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, counts, D.E, offsets, tile_offsets);
  return hipGetLastError();
}

// -------------------------------------------------------------- scatter ----
// Stable rows without order-dependent atomics: one wavefront per chunk of 64
// tokens (lane = token).  Every lane ORs its bit into the LDS mask of each
// expert it picked; the rank of (t, j) inside the chunk's part of expert e's
// group is the number of lower lanes in mask[e].
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ cbase, int T, int E, int k,
                                                 int nchunks, int32_t* __restrict__ perm_src,
                                                 int32_t* __restrict__ inv) {
  extern __shared__ unsigned long long masks[];  // [4][E]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned long long* m = masks + (size_t)w * E;
  for (int e = lane; e < E; e += 64) m[e] = 0ull;
  __syncthreads();
  const int chunk = blockIdx.x * 4 + w;
  const int t = chunk * kChunk + lane;
  const bool valid = chunk < nchunks && t < T;
  if (valid)
    for (int j = 0; j < k; ++j) atomicOr(&m[idx[(size_t)t * k + j]], 1ull << lane);
  __syncthreads();
  if (valid) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      const int rank = __popcll(m[e] & below);
      const int row = offsets[e] + cbase[(size_t)chunk * E + e] + rank;
      if (row < T * k) perm_src[row] = t;  // always true for consistent counts
      inv[(size_t)t * k + j] = row;
    }
  }
}

hipError_t launch_scatter(const Dims& D, const int32_t* idx, const int32_t* offsets, const int32_t* chunk_base, int T,
                          int32_t* perm_src, int32_t* inv, hipStream_t s) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  const size_t lds = (size_t)4 * D.E * sizeof(unsigned long long);
  hipLaunchKernelGGL(k_scatter, dim3((nchunks + 3) / 4), dim3(256), lds, s, idx, offsets, chunk_base, T, D.E, D.k,
                     nchunks, perm_src, inv);
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
// Per expert (one block each): the histogram row goes to LDS and is cleared;
// scanning bins from the top, the bin j with A*E < N*k <= (A+c_j)*E (A =
// tokens above bin j; exact integer tests) holds the score the expert must
// beat to get N*k/E tokens; inside it the estimate is linear:
// q = (j+1)/B - ((N*k - A*E) / (E*c_j)) / B, fp64.
__global__ __launch_bounds__(256) void k_qb_quantile(uint32_t* __restrict__ hist,
                                                     const unsigned long long* __restrict__ count, int E, int B,
                                                     int k, double* __restrict__ q) {
#pragma clang fp contract(off)
  __shared__ uint32_t row[256];
  const unsigned long long N = *count;
  if (N == 0) return;
  const int e = blockIdx.x;
  uint32_t* hr = hist + (size_t)e * B;
  for (int i = threadIdx.x; i < B; i += 256) {
    row[i] = hr[i];
    hr[i] = 0u;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long target = N * (unsigned long long)k;
    const unsigned long long EE = (unsigned long long)E;
    unsigned long long above = 0;
    double qe = 0.0;
    for (int j = B - 1; j >= 0; --j) {
      const unsigned long long c = row[j];
      if (above * EE < target && target <= (above + c) * EE) {
        const double frac = (double)(target - above * EE) / (double)(EE * c);
        qe = (double)(j + 1) / (double)B - frac / (double)B;
        break;
      }
      above += c;
    }
    q[e] = qe;
  }
}

// b_e = fp32(mu - q_e), mu the fp64 mean of q summed in expert order; then the
// token count is cleared.  Keeps the bias when no token was accumulated.
__global__ __launch_bounds__(1024) void k_qb_bias(const double* __restrict__ q, unsigned long long* __restrict__ count,
                                                  int E, float* __restrict__ bias) {
#pragma clang fp contract(off)
  __shared__ double mu_s;
  if (*count == 0) return;
  if (threadIdx.x == 0) {
    double mu = 0.0;
    for (int e = 0; e < E; ++e) mu += q[e];
    mu_s = mu / (double)E;
  }
  __syncthreads();
  const double mu = mu_s;
  for (int e = threadIdx.x; e < E; e += 1024) bias[e] = (float)(mu - q[e]);
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
