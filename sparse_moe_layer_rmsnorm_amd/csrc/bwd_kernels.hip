// Memory-bound kernels of the layer's backward pass (gfx950): operand
// transposes for the weight-gradient products, the padded per-expert K map,
// the GLU, combine, dispatch and gate transposes, and the RMSNorm gradient.
// The products themselves run on the GEMM kernels of gemm_kernels.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// 16 bytes <-> 8 bf16 or 4 fp32 values
template <bool BF16>
MOE_DEV void unpack(const uint4& v, float* f) {
  if constexpr (BF16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
      f[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  } else {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
}
template <bool BF16>
MOE_DEV uint4 pack(const float* f) {
  if constexpr (BF16)
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  else
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

template <bool BF16>
MOE_DEV float ld_act(const void* p, size_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}
template <bool BF16>
MOE_DEV void st_act(void* p, size_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<float*>(p)[i] = v;
}

// ------------------------------------------------------------ transpose ----
// dst[c][col_off + p] = src[row(p)][c] for p < P, c < C, where row(p) =
// gather[colmap[p]] (each map optional: identity when NULL); p whose row is
// negative or >= R gives 0 (pad columns).  64 x 64 tiles through LDS, reads
// coalesced along c, writes along p; blockIdx.z walks a batch of matrices.
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ src, int R, int C, long long ld_src,
                                                   long long src_bstride, const int32_t* __restrict__ gather,
                                                   const int32_t* __restrict__ colmap, int P, E* __restrict__ dst,
                                                   long long ld_dst, long long col_off, long long dst_bstride) {
  __shared__ E tile[64][65];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  src += (size_t)blockIdx.z * src_bstride;
  dst += (size_t)blockIdx.z * dst_bstride;
  const int tid = threadIdx.x;
  {
    const int cl = tid & 63, pg = tid >> 6;
    const int c = c0 + cl;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int pl = pg + 4 * i, p = p0 + pl;
      E v = 0;
      if (p < P && c < C) {
        const int r = colmap ? colmap[p] : p;
        if (r >= 0 && r < R) v = src[(size_t)(gather ? gather[r] : r) * ld_src + c];
      }
      tile[pl][cl] = v;
    }
  }
  __syncthreads();
  const int pl = tid & 63, cg = tid >> 6;
  const int p = p0 + pl;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int cl = cg + 4 * i, c = c0 + cl;
    if (c < C && p < P) dst[(size_t)c * ld_dst + col_off + p] = tile[pl][cl];
  }
}

// Vectorised transposes for the common case (C and P multiples of 64, rows
// and column offsets on 16-byte boundaries): each wavefront reads 8 (bf16) or
// 4 (fp32) source rows as whole 128/256-byte runs and writes whole 128-byte
// runs of destination rows; the tile sits in LDS as dwords with one pad
// dword per row, so that neither phase has bank conflicts beyond two-way.
MOE_DEV int src_row_of(int p, int R, const int32_t* __restrict__ gather, const int32_t* __restrict__ colmap) {
  const int r = colmap ? colmap[p] : p;
  return (r >= 0 && r < R) ? (gather ? gather[r] : r) : -1;
}

// Segment mode (seg_tile non-NULL): the columns p form per-expert segments
// seg_koff[e] .. seg_koff[e+1] (whole 64-column tiles, seg_tile[p / 64] = e,
// -1 past the last); each expert's transposed block [C, pad_e] is stored
// contiguously at seg_koff[e] * C, so that its rows are pad_e long.
MOE_DEV bool seg_dst(const int32_t* __restrict__ seg_koff, const int32_t* __restrict__ seg_tile, int C, int p0,
                     long long& base, long long& ld) {
  const int e = seg_tile[p0 / 64];
  if (e < 0) return false;
  const int s0 = seg_koff[e];
  ld = seg_koff[e + 1] - s0;
  base = (long long)s0 * C - s0;  // + c * ld + p
  return true;
}

__global__ __launch_bounds__(256) void k_transpose_b16(const uint16_t* __restrict__ src, int R, long long ld_src,
                                                       long long src_bstride, const int32_t* __restrict__ gather,
                                                       const int32_t* __restrict__ colmap, uint16_t* __restrict__ dst,
                                                       long long ld_dst, long long col_off, long long dst_bstride,
                                                       const int32_t* __restrict__ seg_koff,
                                                       const int32_t* __restrict__ seg_tile) {
  __shared__ uint32_t tile[64][33];  // row p: 64 bf16 of c as 32 dwords
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64, t = threadIdx.x;
  if (seg_tile && !seg_dst(seg_koff, seg_tile, gridDim.y * 64, p0, col_off, ld_dst)) return;
  src += (size_t)blockIdx.z * src_bstride;
  dst += (size_t)blockIdx.z * dst_bstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + 256 * i, pr = idx >> 3, ch = idx & 7;
    const int sr = src_row_of(p0 + pr, R, gather, colmap);
    const uint4 v = sr >= 0 ? *reinterpret_cast<const uint4*>(src + (size_t)sr * ld_src + c0 + 8 * ch)
                            : make_uint4(0, 0, 0, 0);
    tile[pr][4 * ch + 0] = v.x;
    tile[pr][4 * ch + 1] = v.y;
    tile[pr][4 * ch + 2] = v.z;
    tile[pr][4 * ch + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + 256 * i, pc = idx & 7, cr = idx >> 3;
    const int sh = (cr & 1) * 16;
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (tile[8 * pc + j][cr >> 1] >> sh) & 0xFFFFu;
    *reinterpret_cast<uint4*>(dst + (size_t)(c0 + cr) * ld_dst + col_off + p0 + 8 * pc) =
        make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
  }
}

__global__ __launch_bounds__(256) void k_transpose_b32(const uint32_t* __restrict__ src, int R, long long ld_src,
                                                       long long src_bstride, const int32_t* __restrict__ gather,
                                                       const int32_t* __restrict__ colmap, uint32_t* __restrict__ dst,
                                                       long long ld_dst, long long col_off, long long dst_bstride,
                                                       const int32_t* __restrict__ seg_koff,
                                                       const int32_t* __restrict__ seg_tile) {
  __shared__ uint32_t tile[64][65];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64, t = threadIdx.x;
  if (seg_tile && !seg_dst(seg_koff, seg_tile, gridDim.y * 64, p0, col_off, ld_dst)) return;
  src += (size_t)blockIdx.z * src_bstride;
  dst += (size_t)blockIdx.z * dst_bstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = t + 256 * i, pr = idx >> 4, ch = idx & 15;
    const int sr = src_row_of(p0 + pr, R, gather, colmap);
    const uint4 v = sr >= 0 ? *reinterpret_cast<const uint4*>(src + (size_t)sr * ld_src + c0 + 4 * ch)
                            : make_uint4(0, 0, 0, 0);
    tile[pr][4 * ch + 0] = v.x;
    tile[pr][4 * ch + 1] = v.y;
    tile[pr][4 * ch + 2] = v.z;
    tile[pr][4 * ch + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = t + 256 * i, pc = idx & 15, cr = idx >> 4;
    *reinterpret_cast<uint4*>(dst + (size_t)(c0 + cr) * ld_dst + col_off + p0 + 4 * pc) =
        make_uint4(tile[4 * pc][cr], tile[4 * pc + 1][cr], tile[4 * pc + 2][cr], tile[4 * pc + 3][cr]);
  }
}

// ---------------------------------------------------- padded expert K map ----
// koff[e] = sum over e' < e of pad(n_e'), pad(n) = max(1, ceil(n / 64)) * 64,
// koff[E] the total; colmap[koff[e] + j] = offsets[e] + j for j < n_e, else
// -1, and -1 from koff[E] up to Kt (the host's bound on the total).  One
// block of 1024 threads (E <= 1024).
__global__ __launch_bounds__(1024) void k_pad_map(const int32_t* __restrict__ offsets, int E, int Kt,
                                                  int32_t* __restrict__ koff, int32_t* __restrict__ colmap,
                                                  int32_t* __restrict__ seg_tile) {
  __shared__ int wsum[16];
  __shared__ int base[1024];
  const int i = threadIdx.x, lane = i & 63, w = i >> 6;
  const int n = i < E ? offsets[i + 1] - offsets[i] : 0;
  const int pad = i < E ? max(1, (n + 63) / 64) * 64 : 0;
  int r = pad;  // inclusive wave scan
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(r, o, 64);
    if (lane >= o) r += v;
  }
  if (lane == 63) wsum[w] = r;
  __syncthreads();
  for (int j = 0; j < w; ++j) r += wsum[j];
  base[i] = r - pad;
  if (i < E) koff[i] = r - pad;
  if (i == E - 1) koff[E] = r;
  __syncthreads();
  for (int e = w; e < E; e += 16) {  // one wavefront per expert
    const int b = base[e], off = offsets[e], ne = offsets[e + 1] - off;
    const int pe = max(1, (ne + 63) / 64) * 64;
    for (int j = lane; j < pe; j += 64) colmap[b + j] = j < ne ? off + j : -1;
    for (int j = lane; j < pe / 64; j += 64) seg_tile[b / 64 + j] = e;
  }
  const int tot = base[E - 1] + max(1, (offsets[E] - offsets[E - 1] + 63) / 64) * 64;
  for (int j = tot + i; j < Kt; j += 1024) colmap[j] = -1;
  for (int j = tot / 64 + i; j < Kt / 64; j += 1024) seg_tile[j] = -1;
}

// ------------------------------------------------------------------ GLU ----
// G = silu(P) * Q  ->  dP = dG * Q * silu'(P), dQ = dG * silu(P), with
// silu'(a) = sig(a) (1 + a (1 - sig(a))).  P, Q, dG [R, n] (ld n); dP, dQ at
// rows of ldo elements.  fp32 arithmetic, stored in the activation dtype.
// 16 bytes per thread and operand (n is a multiple of 64).
template <bool BF16>
__global__ __launch_bounds__(256) void k_glu_bwd(const void* __restrict__ P, const void* __restrict__ Q,
                                                 const void* __restrict__ dG, long long R, int n, void* __restrict__ dP,
                                                 void* __restrict__ dQ, int ldo) {
  constexpr int V = BF16 ? 8 : 4;
  const long long total = R * n / V;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long e0 = i * V;
    const long long r = e0 / n;
    const int c = (int)(e0 - r * n);
    const uint4 pa = reinterpret_cast<const uint4*>(P)[i], qa = reinterpret_cast<const uint4*>(Q)[i];
    const uint4 ga = reinterpret_cast<const uint4*>(dG)[i];
    float a[V], u[V], g[V], op[V], oq[V];
    unpack<BF16>(pa, a);
    unpack<BF16>(qa, u);
    unpack<BF16>(ga, g);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float sg = 1.0f / (1.0f + __expf(-a[j]));
      op[j] = g[j] * u[j] * (sg * (1.0f + a[j] * (1.0f - sg)));
      oq[j] = g[j] * a[j] * sg;
    }
    const size_t o = ((size_t)r * ldo + c) / V;
    reinterpret_cast<uint4*>(dP)[o] = pack<BF16>(op);
    reinterpret_cast<uint4*>(dQ)[o] = pack<BF16>(oq);
  }
}

// -------------------------------------------------------------- combine ----
// y_lat[t] = sum_j g_tj Y[inv_tj]  ->  dY[inv_tj] = g_tj dy[t],
// dg_tj = <dy[t], Y[inv_tj]>.  One wavefront per token, 16-byte chunks.
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine_bwd(const void* __restrict__ dy, const void* __restrict__ Y,
                                                     const float* __restrict__ gates, const int32_t* __restrict__ inv,
                                                     int T, int l, int k, void* __restrict__ dY,
                                                     float* __restrict__ dg) {
  constexpr int V = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = 0;
  float my_g = 0.f;
  if (lane < k) {
    my_row = inv[(size_t)t * k + lane];
    my_g = gates[(size_t)t * k + lane];
  }
  const int nc = l / V;
  const uint4* dyr = reinterpret_cast<const uint4*>(dy) + (size_t)t * nc;
  for (int j = 0; j < k; ++j) {
    const int row = __builtin_amdgcn_readlane(my_row, j);
    const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j));
    const uint4* yr = reinterpret_cast<const uint4*>(Y) + (size_t)row * nc;
    uint4* out = reinterpret_cast<uint4*>(dY) + (size_t)row * nc;
    float dot = 0.f;
    for (int c = lane; c < nc; c += 64) {
      float a[V], b[V], o[V];
      unpack<BF16>(dyr[c], a);
      unpack<BF16>(yr[c], b);
#pragma unroll
      for (int q = 0; q < V; ++q) {
        dot += a[q] * b[q];
        o[q] = g * a[q];
      }
      out[c] = pack<BF16>(o);
    }
    dot = wave_sum(dot);
    if (lane == 0) dg[(size_t)t * k + j] = dot;
  }
}

// ------------------------------------------------------------- dispatch ----
// X[r] = z[perm_src[r]]  ->  dz[t] = sum_j dX[inv_tj] (slot order, fp32).
template <bool BF16>
__global__ __launch_bounds__(256) void k_dispatch_bwd(const void* __restrict__ dX, const int32_t* __restrict__ inv,
                                                      int T, int l, int k, void* __restrict__ dz, int ldo) {
  constexpr int V = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my_row = lane < k ? inv[(size_t)t * k + lane] : 0;
  const int nc = l / V;
  for (int c = lane; c < nc; c += 64) {
    float a[V];
#pragma unroll
    for (int q = 0; q < V; ++q) a[q] = 0.f;
    for (int j = 0; j < k; ++j) {
      float b[V];
      unpack<BF16>(reinterpret_cast<const uint4*>(dX)[(size_t)__builtin_amdgcn_readlane(my_row, j) * nc + c], b);
#pragma unroll
      for (int q = 0; q < V; ++q) a[q] += b[q];
    }
    reinterpret_cast<uint4*>(dz)[((size_t)t * ldo) / V + c] = pack<BF16>(a);
  }
}

// ---------------------------------------------------------------- gates ----
// g_j = c s_j / S over the selected experts (S their sum in slot order):
// ds_j = (c / S) dg_j - (1 / S) sum_i dg_i g_i; dl_j = ds_j s_j (1 - s_j).
// The scores are recomputed from the logits by the same sigmoid as the
// forward.  Writes the whole row of Epad columns: dl at the selected
// experts, 0 elsewhere (the bias gets no gradient).  One wavefront per token.
template <bool BF16>
__global__ __launch_bounds__(256) void k_gates_bwd(const float* __restrict__ logits, const int32_t* __restrict__ idx,
                                                   const float* __restrict__ dg, int T, int E, int Epad, int k,
                                                   float scale, void* __restrict__ dl, int ldo) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_e = -1;
  float my_s = 0.f, my_dg = 0.f;
  if (lane < k) {
    my_e = idx[(size_t)t * k + lane];
    my_s = router_sigmoid(logits[(size_t)t * E + my_e]);
    my_dg = dg[(size_t)t * k + lane];
  }
  float S = 0.f;
  for (int j = 0; j < k; ++j) S += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  const float g = scale * my_s / S;
  float A = 0.f;
  for (int j = 0; j < k; ++j) {
    const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), j));
    A += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dg), j)) * gj;
  }
  const float ds = scale * my_dg / S - A / S;
  const float my_dl = ds * my_s * (1.0f - my_s);
  for (int c = lane; c < Epad; c += 64) {
    float v = 0.f;
    for (int j = 0; j < k; ++j)
      if (__builtin_amdgcn_readlane(my_e, j) == c) v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dl), j));
    st_act<BF16>(dl, (size_t)t * ldo + c, v);
  }
}

// -------------------------------------------------------------- RMSNorm ----
// h = gamma x r, r = (mean(x^2) + eps)^-1/2 (fp32, as in the forward):
// dx = r u - x r^3 <u, x> / d with u = gamma dh.  One wavefront per row; r
// is kept for the gamma gradient.
template <bool BF16>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const void* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ dh, int T, int d, float eps,
                                                     void* __restrict__ dx, float* __restrict__ rstd) {
  constexpr int V = BF16 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nc = d / V;
  const uint4* xr = reinterpret_cast<const uint4*>(x) + (size_t)t * nc;
  const float4* dhr = reinterpret_cast<const float4*>(dh + (size_t)t * d);
  const float4* gr = reinterpret_cast<const float4*>(gamma);
  float ss = 0.f, dot = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float a[V];
    unpack<BF16>(xr[c], a);
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const float4 u = dhr[c * (V / 4) + q], gm = gr[c * (V / 4) + q];
      ss += a[4 * q] * a[4 * q] + a[4 * q + 1] * a[4 * q + 1] + a[4 * q + 2] * a[4 * q + 2] + a[4 * q + 3] * a[4 * q + 3];
      dot += gm.x * u.x * a[4 * q] + gm.y * u.y * a[4 * q + 1] + gm.z * u.z * a[4 * q + 2] + gm.w * u.w * a[4 * q + 3];
    }
  }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  const float corr = r * r * r * dot / (float)d;
  uint4* dxr = reinterpret_cast<uint4*>(dx) + (size_t)t * nc;
  for (int c = lane; c < nc; c += 64) {
    float a[V], o[V];
    unpack<BF16>(xr[c], a);
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const float4 u = dhr[c * (V / 4) + q], gm = gr[c * (V / 4) + q];
      o[4 * q] = r * gm.x * u.x - a[4 * q] * corr;
      o[4 * q + 1] = r * gm.y * u.y - a[4 * q + 1] * corr;
      o[4 * q + 2] = r * gm.z * u.z - a[4 * q + 2] * corr;
      o[4 * q + 3] = r * gm.w * u.w - a[4 * q + 3] * corr;
    }
    dxr[c] = pack<BF16>(o);
  }
  if (lane == 0) rstd[t] = r;
}

// dgamma[c] = sum_t dh[t,c] x[t,c] r[t]: slice s of the rows -> part[s][c],
// then the slices are summed in order (deterministic).
template <bool BF16>
__global__ __launch_bounds__(256) void k_dgamma_part(const void* __restrict__ x, const float* __restrict__ dh,
                                                     const float* __restrict__ rstd, int T, int d, int rows_per,
                                                     float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const int t0 = blockIdx.y * rows_per, t1 = min(T, t0 + rows_per);
  float a = 0.f;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) a += dh[(size_t)t * d + c] * ld_act<BF16>(x, (size_t)t * d + c) * rstd[t];
  part[(size_t)blockIdx.y * d + c] = a;
}

__global__ __launch_bounds__(256) void k_sum_slices(const float* __restrict__ part, int S, int n,
                                                    float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  float a = 0.f;
#pragma unroll 16
  for (int s = 0; s < S; ++s) a += part[(size_t)s * n + c];
  out[c] = a;
}

__global__ void k_fill_koff(int32_t* __restrict__ koff, int n, int step, int total) {
  const int j = threadIdx.x;
  if (j <= n) koff[j] = min(j * step, total);
}

// C = sum over the S partials, then stored into the segment that holds the
// row (by_rows) or column; four consecutive columns per thread.
__global__ __launch_bounds__(256) void k_reduce_split(const float4* __restrict__ part, int S, int M, int N,
                                                      const SplitOut o) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;  // float4 index
  const long long n4 = (long long)M * N / 4;
  if (q >= n4) return;
  float4 a = part[q];
  for (int j = 1; j < S; ++j) {
    const float4 v = part[(size_t)j * n4 + q];
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  const int m = (int)(q * 4 / N), n = (int)(q * 4 - (long long)m * N);
  const int key = o.by_rows ? m : n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < o.nseg && key >= o.start[i] && key < o.start[i] + o.len[i]) {
      const int r = o.by_rows ? m - o.start[i] : m, c = o.by_rows ? n : n - o.start[i];
      *reinterpret_cast<float4*>(o.out[i] + (size_t)r * o.ld[i] + c) = a;
    }
  }
}

unsigned blocks_for(long long n, int per_block) {
  long long b = (n + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

}  // namespace

hipError_t launch_fill_koff(int32_t* koff, int n, int step, int total, hipStream_t s) {
  if (n < 1 || n > 255) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fill_koff, dim3(1), dim3(256), 0, s, koff, n, step, total);
  return hipGetLastError();
}

hipError_t launch_reduce_split(const float* part, int S, int M, int N, const SplitOut& o, hipStream_t s) {
  if (N % 4) return hipErrorInvalidValue;
  for (int i = 0; i < o.nseg; ++i)
    if ((!o.by_rows && o.start[i] % 4) || o.ld[i] % 4 || ((uintptr_t)o.out[i] & 15)) return hipErrorInvalidValue;
  const long long n4 = (long long)M * N / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce_split, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(part), S, M, N, o);
  return hipGetLastError();
}

hipError_t launch_transpose(const Dims& D, const void* src, int R, int C, long long ld_src, long long src_bstride,
                            const int32_t* gather, const int32_t* colmap, int P, void* dst, long long ld_dst,
                            long long col_off, long long dst_bstride, int batch, hipStream_t s,
                            const int32_t* seg_koff, const int32_t* seg_tile) {
  if (P <= 0 || C <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((P + 63) / 64, (C + 63) / 64, batch);
  const int V = D.bf16 ? 8 : 4;
  const bool vec = C % 64 == 0 && P % 64 == 0 && ld_src % V == 0 && ld_dst % V == 0 && col_off % V == 0 &&
                   src_bstride % V == 0 && dst_bstride % V == 0 && ((uintptr_t)src & 15) == 0 &&
                   ((uintptr_t)dst & 15) == 0;
  if (seg_tile && !vec) return hipErrorInvalidValue;
  if (vec) {
    if (D.bf16)
      hipLaunchKernelGGL(k_transpose_b16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), R, ld_src,
                         src_bstride, gather, colmap, static_cast<uint16_t*>(dst), ld_dst, col_off, dst_bstride,
                         seg_koff, seg_tile);
    else
      hipLaunchKernelGGL(k_transpose_b32, grid, dim3(256), 0, s, static_cast<const uint32_t*>(src), R, ld_src,
                         src_bstride, gather, colmap, static_cast<uint32_t*>(dst), ld_dst, col_off, dst_bstride,
                         seg_koff, seg_tile);
    return hipGetLastError();
  }
  if (D.bf16)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), R, C, ld_src,
                       src_bstride, gather, colmap, P, static_cast<uint16_t*>(dst), ld_dst, col_off, dst_bstride);
  else
    hipLaunchKernelGGL(k_transpose<uint32_t>, grid, dim3(256), 0, s, static_cast<const uint32_t*>(src), R, C, ld_src,
                       src_bstride, gather, colmap, P, static_cast<uint32_t*>(dst), ld_dst, col_off, dst_bstride);
  return hipGetLastError();
}

hipError_t launch_pad_map(const Dims& D, const int32_t* offsets, int Kt, int32_t* koff, int32_t* colmap,
                          int32_t* seg_tile, hipStream_t s) {
  hipLaunchKernelGGL(k_pad_map, dim3(1), dim3(1024), 0, s, offsets, D.E, Kt, koff, colmap, seg_tile);
  return hipGetLastError();
}

hipError_t launch_glu_bwd(const Dims& D, const void* P, const void* Q, const void* dG, long long R, int n, void* dP,
                          void* dQ, int ldo, hipStream_t s) {
  if (R == 0 || n == 0) return hipSuccess;
  if (n % 64 || ldo % 64) return hipErrorInvalidValue;
  const unsigned g = blocks_for(R * n / (D.bf16 ? 8 : 4), 256 * 2);
  if (D.bf16) hipLaunchKernelGGL(k_glu_bwd<true>, dim3(g), dim3(256), 0, s, P, Q, dG, R, n, dP, dQ, ldo);
  else hipLaunchKernelGGL(k_glu_bwd<false>, dim3(g), dim3(256), 0, s, P, Q, dG, R, n, dP, dQ, ldo);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const Dims& D, const void* dy, const void* Y, const float* gates, const int32_t* inv,
                              int T, void* dY, float* dg, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16) hipLaunchKernelGGL(k_combine_bwd<true>, grid, dim3(256), 0, s, dy, Y, gates, inv, T, D.l, D.k, dY, dg);
  else hipLaunchKernelGGL(k_combine_bwd<false>, grid, dim3(256), 0, s, dy, Y, gates, inv, T, D.l, D.k, dY, dg);
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd(const Dims& D, const void* dX, const int32_t* inv, int T, void* dz, int ldo,
                               hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16) hipLaunchKernelGGL(k_dispatch_bwd<true>, grid, dim3(256), 0, s, dX, inv, T, D.l, D.k, dz, ldo);
  else hipLaunchKernelGGL(k_dispatch_bwd<false>, grid, dim3(256), 0, s, dX, inv, T, D.l, D.k, dz, ldo);
  return hipGetLastError();
}

hipError_t launch_gates_bwd(const Dims& D, const float* logits, const int32_t* idx, const float* dg, int T, int Epad,
                            void* dl, int ldo, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16)
    hipLaunchKernelGGL(k_gates_bwd<true>, grid, dim3(256), 0, s, logits, idx, dg, T, D.E, Epad, D.k, D.routed_scale,
                       dl, ldo);
  else
    hipLaunchKernelGGL(k_gates_bwd<false>, grid, dim3(256), 0, s, logits, idx, dg, T, D.E, Epad, D.k, D.routed_scale,
                       dl, ldo);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const Dims& D, const void* x, const float* gamma, const float* dh, int T, void* dx,
                              float* rstd, float* part, int slices, float* dgamma, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (D.bf16) hipLaunchKernelGGL(k_rmsnorm_bwd<true>, grid, dim3(256), 0, s, x, gamma, dh, T, D.d, D.eps, dx, rstd);
  else hipLaunchKernelGGL(k_rmsnorm_bwd<false>, grid, dim3(256), 0, s, x, gamma, dh, T, D.d, D.eps, dx, rstd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows_per = (T + slices - 1) / slices;
  dim3 g2((D.d + 255) / 256, slices);
  if (D.bf16) hipLaunchKernelGGL(k_dgamma_part<true>, g2, dim3(256), 0, s, x, dh, rstd, T, D.d, rows_per, part);
  else hipLaunchKernelGGL(k_dgamma_part<false>, g2, dim3(256), 0, s, x, dh, rstd, T, D.d, rows_per, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_slices, dim3((D.d + 255) / 256), dim3(256), 0, s, part, slices, D.d, dgamma);
  return hipGetLastError();
}

}  // namespace moe
