// Device helpers shared by the HIP kernels of the LatentMoE layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- bf16 ----
MOE_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
MOE_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// ------------------------------------------------------------- sigmoid ----
// Router score s = 1 / (1 + exp(-l)), every step a separately rounded fp32
// operation so that the result is reproducible bit for bit on any IEEE fp32
// machine:  y = -clamp(l, -30, 30); n = rint(y log2 e);
// r = (y - n ln2_hi) - n ln2_lo (Cody-Waite reduction with ln 2 split after
// 16 significant bits, so n ln2_hi is exact); exp(r) by its degree-7 Taylor
// polynomial in Horner form; e = exp(r) 2^n; s = 1 / (1 + e) (IEEE divide).
MOE_DEV float router_sigmoid(float logit) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;   // fp32(1 / ln 2)
  const float kLn2Hi = 0x1.62e4p-1f;     // ln 2 truncated to 16 significant bits
  const float kLn2Lo = 0x1.7f7d1cp-20f;  // fp32(ln 2 - kLn2Hi)
  const float c7 = 0x1.a01a02p-13f;      // fp32(1/7!)
  const float c6 = 0x1.6c16c2p-10f;      // fp32(1/6!)
  const float c5 = 0x1.111112p-7f;       // fp32(1/5!)
  const float c4 = 0x1.555556p-5f;       // fp32(1/4!)
  const float c3 = 0x1.555556p-3f;       // fp32(1/3!)
  float y = -fminf(fmaxf(logit, -30.0f), 30.0f);
  float n = __builtin_rintf(y * kLog2e);
  float r = (y - n * kLn2Hi) - n * kLn2Lo;
  float p = c7;
  p = p * r + c6;
  p = p * r + c5;
  p = p * r + c4;
  p = p * r + c3;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  float e = __builtin_ldexpf(p, (int)n);
  return 1.0f / (1.0f + e);
}

// Fast router score: the same clamp, then the hardware base-2 exponential
// and reciprocal (v_exp_f32, v_rcp_f32).  It only decides where exact scores
// are needed: every fp32 logit gives |fast_sigmoid - router_sigmoid| <=
// kFastScoreErr (the library's moe_fast_score_error measures the largest
// difference over all 2^32 inputs on the device), and each decision taken
// from a fast score keeps a distance of at least twice that bound from the
// point where the exact score could decide otherwise.
constexpr float kFastScoreErr = 0x1p-20f;
MOE_DEV float fast_sigmoid(float logit) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;
  const float y = -fminf(fmaxf(logit, -30.0f), 30.0f);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y * kLog2e));
}

// Histogram bin of a score over the range [lo, lo + B / scale]:
// clamp(floor(fp32(fp32(s - lo) * scale)), 0, B - 1), scale = fp32(B / (hi -
// lo)); on [0, 1] this is min(B - 1, floor(s * B)) with s*B in fp32.  Scores
// beyond the range fall in the end bins (the clamp is done in fp32 first, so
// no out-of-range float reaches the integer conversion).
MOE_DEV int score_bin(float s, int B, float lo, float scale) {
#pragma clang fp contract(off)
  const float t = floorf((s - lo) * scale);
  const float c = fminf(fmaxf(t, 0.0f), (float)(B - 1));
  return (int)c;
}

// score_bin(router_sigmoid(logit), ...) computed from the fast score: when
// no bin boundary (nor clamp edge) lies within dlt of the fast position x',
// the exact position x = fp32(fp32(s - lo) * scale) falls in the same bin,
// since |x' - x| <= kFastScoreErr * scale + 2^-22 |x| (the roundings of the
// subtraction and the product); dlt keeps four times the first term and
// eight times the second.  Otherwise the exact score decides.
MOE_DEV int score_bin_fast(float logit, int B, float lo, float scale) {
#pragma clang fp contract(off)
  const float x = (fast_sigmoid(logit) - lo) * scale;
  const float dlt = 4.0f * kFastScoreErr * scale + fabsf(x) * 0x1p-19f + 0x1p-19f;
  const float top = (float)(B - 1);
  const float a = fminf(fmaxf(floorf(x - dlt), 0.0f), top);
  const float c = fminf(fmaxf(floorf(x + dlt), 0.0f), top);
  if (a == c) return (int)a;
  return score_bin(router_sigmoid(logit), B, lo, scale);
}

// Orderable key of an fp32 value: a larger float gives a larger key; -0 and
// +0 give the same key.
MOE_DEV uint32_t float_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0) u = 0;  // canonical +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Signed-integer order key of an fp32 value (a larger float gives a larger
// int; -0 sorts just below +0), and its inverse (the map is an involution).
MOE_DEV int32_t float_skey(float v) {
  const int32_t u = __float_as_int(v);
  return u ^ ((u >> 31) & 0x7FFFFFFF);
}
MOE_DEV float skey_float(int32_t k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// --------------------------------------------------------- wave helpers ----
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// DPP row shift of a 64-bit value; lanes whose source falls outside their
// row of 16 keep their own value.
template <int CTRL>
MOE_DEV unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF,
                                             false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

MOE_DEV unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

// Maximum over the 64 lanes, returned to every lane (wave-uniform).  Row
// shifts 1, 2, 4, 8 leave each row's maximum in its lane 15; the four row
// maxima are then read out as scalars.  All lanes must be active.
MOE_DEV unsigned long long wave_max_u64(unsigned long long v) {
  unsigned long long w;
  w = dpp_u64<0x111>(v);  // row_shr:1
  v = w > v ? w : v;
  w = dpp_u64<0x112>(v);  // row_shr:2
  v = w > v ? w : v;
  w = dpp_u64<0x114>(v);  // row_shr:4
  v = w > v ? w : v;
  w = dpp_u64<0x118>(v);  // row_shr:8
  v = w > v ? w : v;
  unsigned long long a = readlane_u64(v, 15), b = readlane_u64(v, 31);
  unsigned long long c = readlane_u64(v, 47), d = readlane_u64(v, 63);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Maximum of a 32-bit value over the 64 lanes, wave-uniform (same scheme).
MOE_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(a, b), max(c, d));
}

// Minimum of a signed 32-bit value over the 64 lanes, wave-uniform.
MOE_DEV int32_t wave_min_i32(int32_t v) {
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xF, 0xF, false));
  const int32_t a = __builtin_amdgcn_readlane(v, 15), b = __builtin_amdgcn_readlane(v, 31);
  const int32_t c = __builtin_amdgcn_readlane(v, 47), d = __builtin_amdgcn_readlane(v, 63);
  return min(min(a, b), min(c, d));
}

// Orders the LDS accesses of one wavefront around an exchange between its
// lanes (a wavefront's LDS instructions execute in issue order, so only the
// compiler has to be kept from moving them).
MOE_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Blocks are handed to the 8 XCDs of the chip round-robin.  Map the
// hardware block id to a logical id so that each XCD works on one contiguous
// range of logical ids [0, n) (a bijection on [0, n) for any n).
MOE_DEV int xcd_remap(int b, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = b & 7, local = b >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}
