// Memory-bound kernels of the layer's backward pass (gfx950): the GLU,
// combine, dispatch and gate transposes (the adjoints of those forward
// steps), the RMSNorm gradient and the split-K partial sums.
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
