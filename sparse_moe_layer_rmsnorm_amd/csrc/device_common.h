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

// Orderable key of an fp32 value: a larger float gives a larger key; -0 and
// +0 give the same key.
MOE_DEV uint32_t float_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0) u = 0;  // canonical +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// Blocks are handed to the 8 XCDs of the chip round-robin.  Map the
// hardware block id to a logical id so that each XCD works on one contiguous
// range of logical ids [0, n) (a bijection on [0, n) for any n).
MOE_DEV int xcd_remap(int b, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = b & 7, local = b >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}
