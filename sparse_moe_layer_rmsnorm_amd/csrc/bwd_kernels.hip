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

// ---------------------------------------------------- padded expert K map ----
// koff[e] = sum over e' < e of pad(n_e'), pad(n) = max(1, ceil(n / 64)) * 64,
// koff[E] the total; colmap[koff[e] + j] = offsets[e] + j for j < n_e, else
// -1, and -1 from koff[E] up to Kt (the host's bound on the total).  One
// block of 1024 threads (E <= 1024).
__global__ __launch_bounds__(1024) void k_pad_map(const int32_t* __restrict__ offsets, int E, int Kt,
                                                  int32_t* __restrict__ koff, int32_t* __restrict__ colmap) {
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
  for (int e = 0; e < E; ++e) {
    const int b = base[e], off = offsets[e], ne = offsets[e + 1] - off;
    const int pe = max(1, (ne + 63) / 64) * 64;
    for (int j = i; j < pe; j += 1024) colmap[b + j] = j < ne ? off + j : -1;
  }
  const int tot = base[E - 1] + max(1, (offsets[E] - offsets[E - 1] + 63) / 64) * 64;
  for (int j = tot + i; j < Kt; j += 1024) colmap[j] = -1;
}

// ------------------------------------------------------------------ GLU ----
// G = silu(P) * Q  ->  dP = dG * Q * silu'(P), dQ = dG * silu(P), with
// silu'(a) = sig(a) (1 + a (1 - sig(a))).  P, Q, dG [R, n] (ld n); dP, dQ at
// rows of ldo elements.  fp32 arithmetic, stored in the activation dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void k_glu_bwd(const void* __restrict__ P, const void* __restrict__ Q,
                                                 const void* __restrict__ dG, long long R, int n, void* __restrict__ dP,
                                                 void* __restrict__ dQ, int ldo) {
  const long long total = R * n;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long r = i / n;
    const int c = (int)(i - r * n);
    const float a = ld_act<BF16>(P, i), u = ld_act<BF16>(Q, i), g = ld_act<BF16>(dG, i);
    const float sg = 1.0f / (1.0f + __expf(-a));
    const size_t o = (size_t)r * ldo + c;
    st_act<BF16>(dP, o, g * u * (sg * (1.0f + a * (1.0f - sg))));
    st_act<BF16>(dQ, o, g * a * sg);
  }
}

// -------------------------------------------------------------- combine ----
// y_lat[t] = sum_j g_tj Y[inv_tj]  ->  dY[inv_tj] = g_tj dy[t],
// dg_tj = <dy[t], Y[inv_tj]>.  One wavefront per token.
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine_bwd(const void* __restrict__ dy, const void* __restrict__ Y,
                                                     const float* __restrict__ gates, const int32_t* __restrict__ inv,
                                                     int T, int l, int k, void* __restrict__ dY,
                                                     float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = 0;
  float my_g = 0.f;
  if (lane < k) {
    my_row = inv[(size_t)t * k + lane];
    my_g = gates[(size_t)t * k + lane];
  }
  for (int j = 0; j < k; ++j) {
    const int row = __builtin_amdgcn_readlane(my_row, j);
    const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_g), j));
    float dot = 0.f;
    for (int c = lane; c < l; c += 64) {
      const float v = ld_act<BF16>(dy, (size_t)t * l + c);
      dot += v * ld_act<BF16>(Y, (size_t)row * l + c);
      st_act<BF16>(dY, (size_t)row * l + c, g * v);
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
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my_row = lane < k ? inv[(size_t)t * k + lane] : 0;
  for (int c = lane; c < l; c += 64) {
    float a = 0.f;
    for (int j = 0; j < k; ++j) a += ld_act<BF16>(dX, (size_t)__builtin_amdgcn_readlane(my_row, j) * l + c);
    st_act<BF16>(dz, (size_t)t * ldo + c, a);
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
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t o = (size_t)t * d;
  float ss = 0.f, dot = 0.f;
  for (int c = lane; c < d; c += 64) {
    const float v = ld_act<BF16>(x, o + c);
    ss += v * v;
    dot += gamma[c] * dh[o + c] * v;
  }
  ss = wave_sum(ss);
  dot = wave_sum(dot);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  const float corr = r * r * r * dot / (float)d;
  for (int c = lane; c < d; c += 64) {
    const float v = ld_act<BF16>(x, o + c);
    st_act<BF16>(dx, o + c, r * gamma[c] * dh[o + c] - v * corr);
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
  for (int t = t0; t < t1; ++t) a += dh[(size_t)t * d + c] * ld_act<BF16>(x, (size_t)t * d + c) * rstd[t];
  part[(size_t)blockIdx.y * d + c] = a;
}

__global__ __launch_bounds__(256) void k_sum_slices(const float* __restrict__ part, int S, int n,
                                                    float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  float a = 0.f;
  for (int s = 0; s < S; ++s) a += part[(size_t)s * n + c];
  out[c] = a;
}

unsigned blocks_for(long long n, int per_block) {
  long long b = (n + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

}  // namespace

hipError_t launch_transpose(const Dims& D, const void* src, int R, int C, long long ld_src, long long src_bstride,
                            const int32_t* gather, const int32_t* colmap, int P, void* dst, long long ld_dst,
                            long long col_off, long long dst_bstride, int batch, hipStream_t s) {
  if (P <= 0 || C <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((P + 63) / 64, (C + 63) / 64, batch);
  if (D.bf16)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), R, C, ld_src,
                       src_bstride, gather, colmap, P, static_cast<uint16_t*>(dst), ld_dst, col_off, dst_bstride);
  else
    hipLaunchKernelGGL(k_transpose<uint32_t>, grid, dim3(256), 0, s, static_cast<const uint32_t*>(src), R, C, ld_src,
                       src_bstride, gather, colmap, P, static_cast<uint32_t*>(dst), ld_dst, col_off, dst_bstride);
  return hipGetLastError();
}

hipError_t launch_pad_map(const Dims& D, const int32_t* offsets, int Kt, int32_t* koff, int32_t* colmap,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_pad_map, dim3(1), dim3(1024), 0, s, offsets, D.E, Kt, koff, colmap);
  return hipGetLastError();
}

hipError_t launch_glu_bwd(const Dims& D, const void* P, const void* Q, const void* dG, long long R, int n, void* dP,
                          void* dQ, int ldo, hipStream_t s) {
  if (R == 0 || n == 0) return hipSuccess;
  const unsigned g = blocks_for(R * n, 256 * 4);
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
