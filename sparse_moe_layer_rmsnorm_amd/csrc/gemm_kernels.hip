// MFMA GEMMs of the LatentMoE layer on gfx950 (CDNA4).
//
// Forward products, y = a W^T with both operands K-contiguous (activation
// rows and PyTorch-layout [out, in] weight rows), fp32 accumulation:
//   * gemm_h:      h [T,d] against [W_r | W_sg,W_su | W_dn] -> fp32 router
//                  logits, the shared GLU hidden G = silu(h W_sg^T)*(h W_su^T)
//                  and the latent z = h W_dn^T in one launch (one pass of h);
//   * expert_up:   per expert, its dispatched rows X against W_g[e], W_u[e]
//                  with the GLU in the epilogue -> H (optionally also the
//                  pre-activations, or H quantised to MXFP8);
//   * expert_down: per expert, H rows against W_d[e] -> Y;
//   * gemm_out:    [G | y_lat] against [W_sd | W_up] (one K loop over both
//                  parts) -> out, so the shared and routed paths are summed in
//                  the fp32 accumulators;
//   * expert_mx / expert_mx4: expert_up / expert_down with MXFP8 activations
//                  against MXFP8 or MXFP4 weights (v_mfma_scale f8f6f4), and
//                  mx_quant, the per-32-column quantiser that feeds them.
// Backward products:
//   * dense_nt / expert_nt: the forward layout with a plain store epilogue,
//                  recomputing the GLU pre-activations h W_sg^T, h W_su^T and
//                  X W_g[e]^T, X W_u[e]^T when they were not kept;
// and, with K-major operands (see Pipe):
//   * dgrad:       dX = dY W with W K-major ([out, in] read along out), dense
//                  or per expert, several operands concatenated along K;
//   * wgrad_km:    dW = dY^T X, contracting over tokens, both operands
//                  token-major, per expert segment of the dispatch order.
// (Width separation and the shared/routed dual path: architecture paragraph
// and Tab 1 of the "Kimi K3 MoE lightweight replica demo" article; the expert
// GLUs as batched matmuls per expert group: capsule 20 of the "Pretraining a
// Mini Kimi K3" review; 4-bit expert weights against 8-bit activations:
// fourth-waste section of the "K3 tops open source" blog, read as the OCP
// MXFP4 / MXFP8 block formats.)
//
// Execution: persistent blocks of 4 wavefronts.  Block b runs on XCD b%8 and
// walks a contiguous range of the logical tile order that belongs to its XCD,
// so the tiles in flight on one XCD share operands in that XCD's L2.  The K
// loops of a block's consecutive tiles form one continuous stream of 128-byte
// K stages through an NS-deep ring of LDS buffers: stages are filled with
// global_load_lds_dwordx4 (global -> LDS DMA, no registers) NS-1 stages ahead,
// also across tile boundaries, so a tile's first loads are in flight while the
// previous tile still computes.  Tile metadata comes from kernel arguments or
// scalar loads, so the stage DMA is the only vector-memory load in the loop
// and the explicit vmcnt waits stay exact.
//
// MFMA: bf16 v_mfma_f32_16x16x32_bf16; fp32 four v_mfma_f32_16x16x4_f32 per
// 16-byte fragment.  The weight fragment is the MFMA's first operand, so each
// lane's accumulators hold 4 consecutive output columns of one row.  LDS rows
// are 128 bytes; 16-byte chunk c of row r sits at position c ^ (r % 8).  A
// ds_read_b128 is served 16 lanes per LDS cycle (64 banks of 4 bytes) in lane
// groups that are not 16 consecutive lanes (measured: the variant that also
// flips chunk bit 0 for rows 8..15 costs twice the cycles); with this
// placement each group of a fragment read hits 16 distinct 16-byte bank slots.
#include <cstring>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// EPI_GLU_MX: EPI_GLU whose output is also quantised to MXFP8 (E4M3 + E8M0
// per 32 columns) in the epilogue.
enum EpiKind { EPI_F32 = 0, EPI_STORE = 1, EPI_GLU = 2, EPI_GLU_MX = 3 };
constexpr bool is_glu(int kind) { return kind == EPI_GLU || kind == EPI_GLU_MX; }


template <bool BF16>
MOE_DEV void mfma_chunk(f32x4_t& acc, const uint4& w, const uint4& a) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w), __builtin_bit_cast(bf16x8_t, a),
                                                   acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), __uint_as_float(a.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), __uint_as_float(a.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), __uint_as_float(a.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), __uint_as_float(a.w), acc, 0, 0, 0);
  }
}

// LDS address (32-bit) of a pointer into a __shared__ array.
MOE_DEV uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte-per-lane global -> LDS DMA load (global_load_lds_dwordx4): lane
// i of the wavefront writes LDS bytes [lds + 16 i, lds + 16 i + 16).  `lds`
// must be wave-uniform.  Issued from inline asm so that the compiler does not
// add a wait for all outstanding loads before every LDS read; the stream loop
// waits for its own loads explicitly.
MOE_DEV void lds_dma16(const char* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}


// Wait until at most N vector-memory operations of this wavefront are
// outstanding.  Loads complete in issue order, so with N = the number of DMA
// loads issued after a stage, that stage has landed in LDS (stores still in
// flight can only lengthen the wait).
template <int N>
MOE_DEV void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

MOE_DEV void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding) for lgkmcnt(0) with vmcnt and expcnt
// left at their maxima, i.e. no wait on them.
constexpr int kLgkmcnt0 = 0xC07F;

// Scalar (SMEM) load of wave-uniform tile metadata written by an earlier kernel.
MOE_DEV int2 scalar_load2(const int2* p, int i) {
  const unsigned long long v = *((const __attribute__((address_space(4))) unsigned long long*)p + i);
  return make_int2((int)(uint32_t)v, (int)(uint32_t)(v >> 32));
}
MOE_DEV int scalar_load(const int32_t* p, int i) {
  return *((const __attribute__((address_space(4))) int32_t*)p + i);
}

// A wave-uniform pointer read into scalar registers.  Per-lane choices
// between two kernel-argument pointers are made on these values, so the
// compiler cannot turn them into a vector load through a per-lane argument
// address (such a load would need a wait on every DMA load in flight).
MOE_DEV const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}
MOE_DEV int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
MOE_DEV long long uniform_ll(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}

// Block-scaled element conversion (MXFP8 / MXFP4) is the hardware's: the
// value is scaled by the block's power of two in fp32 (exact), clamped to
// +-448 (v_cvt_pk_fp8_f32 does not saturate: 464 and above become NaN) and
// converted by v_cvt_pk_fp8_f32, which rounds to nearest even; E2M1 through
// v_cvt_scalef32_pk_fp4_f32 with scale 1, which rounds to nearest even and
// saturates at 6 by itself (both measured on gfx950 over every finite bf16
// value at 11 scales: identical to the reference rounding).
MOE_DEV uint32_t e4m3x4(float a, float b, float c, float d) {
  auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true);
}
MOE_DEV uint32_t e2m1x8(const float* v) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
  return r;
}

// Source of K rows that lie past an operand's end (read by the stage DMA in
// place of a row): 1 KB, never written, zero from load.
__device__ __attribute__((aligned(16))) uint4 g_zero_row[64] = {};

// Block tile BM x BN over WM x WN wavefronts, NS LDS stages of RB K-bytes
// per row (64 or 128), BPC blocks per CU.
//
// LDS layout of a stage: BM + BN rows of RB bytes (A rows, then weight rows).
// 16-byte chunk c of row r sits at chunk position c ^ sw(r): sw = r % 8 for
// 128-byte rows, (r / 2) % 4 for 64-byte rows.  A ds_read_b128 is served 16
// lanes per LDS cycle (64 banks of 4 bytes) in lane groups that are not 16
// consecutive lanes (measured: placing rows 8..15 with chunk bit 0 flipped
// costs twice the cycles); with these placements the 16 lanes of a group that
// read one fragment (16 rows, one logical chunk) hit 16 distinct bank slots.
//
// Stage filling: 1 KB DMA slots (RB = 128: 8 rows of 8 chunks; RB = 64: 16
// rows of 4 chunks); thread (wave w of NW, lane) fills slots i*NW + w, i < L,
// lane l writing chunk position l % (RB/16) of its row, i.e. logical chunk
// (l % (RB/16)) ^ sw(row).
//
// K-major operands (KM bit 0: A, bit 1: B).  Such an operand is stored with
// K as its rows and the tile's M (or N) columns contiguous, e.g. a token-major
// activation in a product that contracts over tokens.  Its region of a stage
// holds KR = RB / element-bytes K rows of P = BM (BN) * element-bytes bytes,
// 16-byte chunk c of row r at position c ^ swzk(r), and fragments are read
// with ds_read_b64_tr_b16 (bf16): lane s of each 16-lane group addresses row
// s / 4 and columns 4 (s % 4) .. + 3 of a 4 x 16 block, and lane i receives
// column i of the block's 4 rows (measured on gfx950), i.e. the MFMA operand
// layout of 16 rows (columns here) by 4 consecutive K values.  fp32 K-major
// fragments are four ds_read_b32 per lane.  The swizzle spreads the rows one
// fragment read touches at once (bf16: rows r % 4 and r / 8 odd or even; fp32:
// the 4 lane groups' rows) over distinct bank slots.
template <int BM_, int BN_, int WM_, int WN_, int NS_, int RB_, int BPC_, bool BF16, int KM_ = 0>
struct Pipe {
  static constexpr int BM = BM_, BN = BN_, NS = NS_, RB = RB_, BPC = BPC_, KM = KM_;
  static constexpr int WM = WM_, WN = WN_, NW = WM * WN;
  static constexpr int THREADS = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 16, NI = WTN / 16;
  static constexpr int KK = RB / 64;                 // 64-byte K steps (one MFMA K each) per stage
  static constexpr int CPR = RB / 16;                // 16-byte chunks per row
  static constexpr int A_BYTES = BM * RB;
  static constexpr int STAGE = (BM + BN) * RB;
  static constexpr int LDS = NS * STAGE;
  static constexpr int L = STAGE / 1024 / NW;  // DMA slots per thread per stage
  static_assert(RB == 64 || RB == 128, "64- or 128-byte stage rows");
  static_assert(STAGE % (1024 * NW) == 0, "stage must split into 1 KB slots over the wavefronts");
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  static_assert(LDS * BPC <= 160 * 1024, "LDS per CU");
  using Acc = f32x4_t[MI][NI];
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int KR = RB / ES;                 // K rows of a K-major region per stage
  static constexpr int PA = BM * ES, PB = BN * ES;   // row bytes of K-major A / B regions
  static constexpr int LA = A_BYTES / (1024 * NW);   // DMA slots of the A region per thread
  static_assert(KM == 0 || (A_BYTES % (1024 * NW) == 0 && PA >= 128 && PB >= 128 && PA <= 1024 && PB <= 1024),
                "K-major regions: whole slots per wavefront, 128- to 1024-byte rows");

  MOE_DEV static int wave_id() { return threadIdx.x >> 6; }

  MOE_DEV static int swz(int row) { return RB == 128 ? (row & 7) : ((row >> 1) & 3); }
  MOE_DEV static int lds_off(int row, int chunk) { return row * RB + ((chunk ^ swz(row)) << 4); }
  MOE_DEV static int slot_row(int i, int wave, int lane) { return (i * NW + wave) * (1024 / RB) + lane / CPR; }
  MOE_DEV static int slot_chunk(int row, int lane) { return (lane % CPR) ^ swz(row); }

  template <int P>
  MOE_DEV static int swzk(int row) {
    if constexpr (BF16) return (2 * ((row & 3) | (((row >> 3) & 1) << 2))) & (P / 16 - 1);
    else return (((row >> 2) & 3) << 2) & (P / 16 - 1);
  }
  template <int P>
  MOE_DEV static int km_off(int row, int colbyte) {
    return row * P + (((colbyte >> 4) ^ swzk<P>(row)) << 4) + (colbyte & 15);
  }
  // DMA slot mapping of a K-major region: lane -> K row of the stage and the
  // logical byte offset (within the tile's columns) of its 16-byte chunk.
  template <int P>
  MOE_DEV static int km_slot_row(int ls, int lane) { return ls * (1024 / P) + lane / (P / 16); }
  template <int P>
  MOE_DEV static int km_slot_colbyte(int row, int lane) { return ((lane % (P / 16)) ^ swzk<P>(row)) << 4; }

  // Fragment of a K-major region: columns col0 .. col0 + 15, 64-byte K step kk.
  template <int P>
  MOE_DEV static uint4 frag_km(const char* region, int col0, int kk) {
    const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
    if constexpr (BF16) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      const int r0 = kk * 32 + 8 * g + (s >> 2), cb = 2 * col0 + 8 * (s & 3);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(region + km_off<P>(r0, cb)));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(region + km_off<P>(r0 + 4, cb)));
      const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
      return make_uint4(a.x, a.y, b.x, b.y);
    } else {
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = *reinterpret_cast<const uint32_t*>(region + km_off<P>(kk * 16 + 4 * g + j, 4 * (col0 + s)));
      return make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  MOE_DEV static uint4 frag_a(const char* cur, int row0, int ch, int kk) {
    if constexpr (KM & 1) return frag_km<PA>(cur, row0, kk);
    else return *reinterpret_cast<const uint4*>(cur + lds_off(row0 + (threadIdx.x & 15), ch));
  }
  MOE_DEV static uint4 frag_b(const char* cur, int row0, int ch, int kk) {
    if constexpr (KM & 2) return frag_km<PB>(cur + A_BYTES, row0, kk);
    else return *reinterpret_cast<const uint4*>(cur + A_BYTES + lds_off(row0 + (threadIdx.x & 15), ch));
  }

  // All fragment reads of the stage are issued before the first MFMA, so
  // the wavefront waits for LDS once per stage rather than once per group.
  MOE_DEV static void compute(const char* cur, Acc& acc) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    if constexpr ((MI + NI) * KK > 16) {  // large wave tiles: one 64-byte K step at a time (registers)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int ch = kk * 4 + (lane >> 4);
        uint4 af[MI], wf[NI];
        // read in first-use order (row fragment 0, every weight fragment, the
        // other row fragments) so each MFMA group waits only for its own reads
        af[0] = frag_a(cur, wm * WTM, ch, kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) wf[ni] = frag_b(cur, wn * WTN + ni * 16, ch, kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 1; mi < MI; ++mi) af[mi] = frag_a(cur, wm * WTM + mi * 16, ch, kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) mfma_chunk<BF16>(acc[mi][ni], wf[ni], af[mi]);
      }
      return;
    }
    if constexpr (BF16 && KM == 3) {
      // Both operands K-major: two transposed reads per fragment, 2 (MI+NI)
      // reads per K step, more than lgkmcnt can count at once.  The next K
      // step's reads are interleaved with this step's MFMAs (two reads per
      // MFMA) instead of all being issued up front.
      uint4 af[KK][MI], wf[KK][NI];
      auto load = [&](int kk) {
        const int ch = kk * 4 + (lane >> 4);
        af[kk][0] = frag_a(cur, wm * WTM, ch, kk);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) wf[kk][ni] = frag_b(cur, wn * WTN + ni * 16, ch, kk);
#pragma unroll
        for (int mi = 1; mi < MI; ++mi) af[kk][mi] = frag_a(cur, wm * WTM + mi * 16, ch, kk);
      };
      load(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) load(kk + 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) mfma_chunk<BF16>(acc[mi][ni], wf[kk][ni], af[kk][mi]);
        if (kk + 1 < KK) {
#pragma unroll
          for (int i = 0; i < MI * NI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    uint4 af[KK][MI], wf[KK][NI];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {  // in first-use order, as above
      const int ch = kk * 4 + (lane >> 4);
      af[kk][0] = frag_a(cur, wm * WTM, ch, kk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) wf[kk][ni] = frag_b(cur, wn * WTN + ni * 16, ch, kk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 1; mi < MI; ++mi) af[kk][mi] = frag_a(cur, wm * WTM + mi * 16, ch, kk);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) mfma_chunk<BF16>(acc[mi][ni], wf[kk][ni], af[kk][mi]);
  }

  MOE_DEV static void zero(Acc& acc) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Wait for a stage after which `after` further stages were issued.
  MOE_DEV static void wait_stage(int after) {
    if (after <= 0) wait_vmcnt<0>();
    else if (after == 1) wait_vmcnt<L>();
    else if (after == 2 || 3 * L > 63) wait_vmcnt<2 * L>();
    else wait_vmcnt<(3 * L > 63 ? 2 * L : 3 * L)>();
  }

  // Row-major store of 4 consecutive columns.
  MOE_DEV static void store4(void* out, size_t idx, float v0, float v1, float v2, float v3) {
    if constexpr (BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v0, v1, v2, v3);
    }
  }

  // Epilogues.  Lane holds rows m = wm*WTM + mi*16 + lane%16 and columns
  // n = wn*WTN + ni*16 + 4*(lane/16) + r (r = 0..3) of the block tile.
  //   EPI_F32:   fp32 store (+ per-column offset, read from LDS), columns < N only.
  //   EPI_STORE: store in the activation dtype (N a multiple of 4).
  //   EPI_GLU:   tile columns alternate 16 gate / 16 up; output column
  //              n0/2 + 16*(c/32) + c%16 gets silu(gate) * up.
  // bf16 outputs of two adjacent 16-column blocks as one 16-byte store per
  // lane: lanes l and l^16 (column quads q, q^1) swap one block's quad, so
  // an even-q lane holds columns 4q..4q+7 of the first block and an odd-q
  // lane columns 4(q-1)..4q+3 of the second.  Every lane takes part in the
  // swap; the stores are then masked.  c0 is the first block's first column.
  MOE_DEV static void store_pair(void* out, size_t orow, int c0, int N, bool row_ok, const float (&x)[4],
                                 const float (&y)[4]) {
    const int lane = threadIdx.x & 63, q = (lane >> 4) & 3;
    const bool odd = q & 1;
    const uint32_t a0 = pack_bf16x2(x[0], x[1]), a1 = pack_bf16x2(x[2], x[3]);
    const uint32_t b0 = pack_bf16x2(y[0], y[1]), b1 = pack_bf16x2(y[2], y[3]);
    const uint32_t r0 = (uint32_t)__shfl_xor((int)(odd ? a0 : b0), 16, 64);
    const uint32_t r1 = (uint32_t)__shfl_xor((int)(odd ? a1 : b1), 16, 64);
    const uint4 v = odd ? make_uint4(r0, r1, b0, b1) : make_uint4(a0, a1, r0, r1);
    const int c = c0 + (odd ? 16 + 4 * (q - 1) : 4 * q);
    if (row_ok && c < N) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + orow + c) = v;
  }

  // EPI_GLU with keep_g / keep_u (wave-uniform, nullable): the gate and up
  // pre-activations are stored too, at the same place as the output.
  // MXFP8 quantisation of one 32-column block of a GLU output row (the two
  // 16-column halves x, y of store_pair, c0 a multiple of 32): the values
  // are rounded to bf16 as stored, the block maximum is taken over the 4
  // lanes of the row, then each lane converts its 8 values.  q8 rows of N
  // bytes, qs rows of N / 32 scale bytes.
  MOE_DEV static void mx8_block(void* q8, void* qs, size_t row, int c0, int N, bool row_ok, const float (&x)[4],
                                const float (&y)[4]) {
    const int lane = threadIdx.x & 63, q = (lane >> 4) & 3;
    const uint32_t p[4] = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(y[0], y[1]),
                           pack_bf16x2(y[2], y[3])};
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(p[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(p[j] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int byte = 0;
    if (amax > 0.f) {
      int e;
      (void)frexpf(amax, &e);
      byte = min(254, max(0, e - 1 - 8 + 127));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ldexpf(v[j], 127 - byte);
    const uint32_t w0 = e4m3x4(v[0], v[1], v[2], v[3]), w1 = e4m3x4(v[4], v[5], v[6], v[7]);
    if (row_ok && c0 < N) {
      uint8_t* d = static_cast<uint8_t*>(q8) + row * (size_t)N + c0;
      *reinterpret_cast<uint32_t*>(d + 4 * q) = w0;
      *reinterpret_cast<uint32_t*>(d + 16 + 4 * q) = w1;
      if (q == 0) static_cast<uint8_t*>(qs)[row * (size_t)(N / 32) + c0 / 32] = (uint8_t)byte;
    }
  }

  // EPI_GLU_MX: keep_g / keep_u are the MXFP8 bytes and scale bytes of the output.
  template <int KIND>
  MOE_DEV static void epilogue(const Acc& acc, int rows_valid, int n0, int N, void* out, int ldo, size_t row_base,
                               const __attribute__((address_space(3))) float* col_off, void* keep_g = nullptr,
                               void* keep_u = nullptr) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    static_assert(KIND != EPI_GLU_MX || (BF16 && NI % 4 == 0), "MXFP8 epilogue: paired bf16 stores only");
    if constexpr (BF16 && KIND != EPI_F32 && NI % 4 == 0) {  // paired 16-byte stores (N is a multiple of 64)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int m = wm * WTM + mi * 16 + (lane & 15);
        const bool row_ok = m < rows_valid;
        const size_t orow = (row_base + (size_t)(row_ok ? m : 0)) * (size_t)ldo;
        if constexpr (is_glu(KIND)) {
#pragma unroll
          for (int p = 0; p < NI / 2; p += 2) {
            float o[2][4], gk[2][4], uk[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4_t g = acc[mi][2 * (p + h)], u = acc[mi][2 * (p + h) + 1];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                o[h][r] = g[r] * u[r] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[r]));
                gk[h][r] = g[r];
                uk[h][r] = u[r];
              }
            }
            const int c0 = n0 / 2 + ((wn * WTN) / 32 + p) * 16;
            store_pair(out, orow, c0, N, row_ok, o[0], o[1]);
            if constexpr (KIND == EPI_GLU_MX) {
              mx8_block(keep_g, keep_u, row_base + (size_t)(row_ok ? m : 0), c0, N, row_ok, o[0], o[1]);
            } else if (keep_g) {
              store_pair(keep_g, orow, c0, N, row_ok, gk[0], gk[1]);
              store_pair(keep_u, orow, c0, N, row_ok, uk[0], uk[1]);
            }
          }
        } else {
#pragma unroll
          for (int ni = 0; ni < NI; ni += 2) {
            const float x[4] = {acc[mi][ni][0], acc[mi][ni][1], acc[mi][ni][2], acc[mi][ni][3]};
            const float y[4] = {acc[mi][ni + 1][0], acc[mi][ni + 1][1], acc[mi][ni + 1][2], acc[mi][ni + 1][3]};
            store_pair(out, orow, n0 + wn * WTN + ni * 16, N, row_ok, x, y);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int m = wm * WTM + mi * 16 + (lane & 15);
      if (m >= rows_valid) continue;
      const size_t orow = (row_base + (size_t)m) * (size_t)ldo;
      if constexpr (KIND == EPI_GLU) {
#pragma unroll
        for (int p = 0; p < NI / 2; ++p) {
          const f32x4_t g = acc[mi][2 * p], u = acc[mi][2 * p + 1];
          const int c = n0 / 2 + ((wn * WTN) / 32 + p) * 16 + 4 * (lane >> 4);
          if (c >= N) continue;
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = g[r] * u[r] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[r]));
          store4(out, orow + c, o[0], o[1], o[2], o[3]);
          if (keep_g) {
            store4(keep_g, orow + c, g[0], g[1], g[2], g[3]);
            store4(keep_u, orow + c, u[0], u[1], u[2], u[3]);
          }
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int c = n0 + wn * WTN + ni * 16 + 4 * (lane >> 4);
          const f32x4_t v = acc[mi][ni];
          if constexpr (KIND == EPI_F32) {
            float* o = static_cast<float*>(out) + orow;
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = v[r] + (col_off && c + r < N ? col_off[c + r] : 0.f);
            if (c + 3 < N && ((ldo | n0) & 3) == 0 && ((uintptr_t)out & 15) == 0) {  // one 16-byte store
              *reinterpret_cast<float4*>(o + c) = make_float4(w[0], w[1], w[2], w[3]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (c + r < N) o[c + r] = w[r];
            }
          } else {
            if (c < N) store4(out, orow + c, v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
};

// A tile of the logical order: first output row, rows in use, n-tile, and the
// segment (dense) or expert (grouped) it belongs to.  Wave-uniform.
struct Tile {
  int row0, rows, nt, sel;
};

// The persistent stream over this block's tiles.  Prob supplies total(),
// kt(), tile(logical), sources(tile, src), issue(src, ks, lds) and
// epilogue(tile, acc).
template <class Pp, class Prob>
MOE_DEV void stream(const Prob& prob, char* smem) {
  const int G = gridDim.x, b = blockIdx.x;
  const int x = b & 7, q = b >> 3, Gx = G >> 3;  // the grid is a multiple of 8
  const int total_tiles = prob.total();
  const int per = (total_tiles + 7) >> 3;
  const int lo = x * per, hi = min(total_tiles, lo + per);
  const int span = hi - lo - q;
  const int my_n = span > 0 ? (span + Gx - 1) / Gx : 0;
  if (my_n <= 0) return;
  const int KT = prob.kt();
  const int total = my_n * KT;
  const uint32_t lds0 = lds_addr(smem) + Pp::wave_id() * 1024;

  typename Prob::template SrcT<Pp::L> src;
  int iss_j = 0, iss_ks = 0, issued = 0;
  prob.sources(prob.tile(lo + q), src);
  auto issue = [&]() {
    const uint32_t base = lds0 + (uint32_t)((issued % Pp::NS) * Pp::STAGE);
    prob.issue(src, iss_ks, base);
    ++issued;
    if (++iss_ks == KT) {
      iss_ks = 0;
      if (++iss_j < my_n) prob.sources(prob.tile(lo + q + iss_j * Gx), src);
    }
  };
  for (int s = 0; s < Pp::NS - 1; ++s)
    if (issued < total) issue();

  typename Pp::Acc acc;
  Pp::zero(acc);
  int cj = 0, cks = 0;
  Tile ct = prob.tile(lo + q);
  for (int g = 0; g < total; ++g) {
    Pp::wait_stage(issued - g - 1);
    block_barrier();
    if (issued < total) issue();
    // Prob::kSettleScalar: wait for any scalar load still in flight before
    // the fragment reads.  Scalar loads share lgkmcnt with LDS reads and
    // return out of order, so while one may be pending the compiler waits for
    // all 16 fragment reads before the first MFMA; with none pending it waits
    // for just the fragments each MFMA group needs, and the later reads land
    // under the first MFMAs (the dense GEMMs gain 2-3%; the grouped ones,
    // whose gather indices come by scalar loads just before, lose).
    if constexpr (Prob::kSettleScalar) __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    Pp::compute(smem + (g % Pp::NS) * Pp::STAGE, acc);
    if (++cks == KT) {
      prob.epilogue(ct, acc);
      Pp::zero(acc);
      cks = 0;
      if (++cj < my_n) ct = prob.tile(lo + q + cj * Gx);
    }
  }
}

// ------------------------------------------------------------ dense GEMMs --
struct DenseSeg {
  const char* B[2];   // weight rows of K part 0 / 1 (gate rows for a GLU)
  const char* Bu[2];  // up rows for a GLU (part 0 only)
  int N;              // output columns
  int ntiles;
  int kind;
  void* out;
  int ldo;
  const float* col_off;  // per-column offset (EPI_F32), at most kMaxColOff columns
  void* keep[2];         // EPI_GLU: gate / up pre-activations also stored (nullable)
};

constexpr int kMaxColOff = 1024;

struct DenseArgs {
  const char* A[2];
  int lda_bytes[2];
  int ldb_bytes[2];
  int kt[2];  // stages per K part
  int M, m_tiles;
  int nseg, total_ntiles;
  DenseSeg seg[3];
};

// Logical tile order: kNSplit column ranges one after the other, each over
// all m-tiles in groups of kGroupM m-tiles (m fastest inside a group).  The
// 8 XCDs take consecutive eighths of this order, so with two column ranges
// each XCD's L2 serves a quarter of the rows and half of the weights (8.7 MB
// per XCD at the replica h GEMM instead of 11.4 MB for an eighth of the rows
// and all the weights).  Measured on the replica h GEMM (8192 x 4608 x 1024):
// 100 us with one range and groups of 8, 91 us with groups of 2, 89 us with
// two ranges (paired runs on one box); four ranges or groups of 64 are slower.
constexpr int kGroupM = 2;
constexpr int kNSplit = 2;

// Logical tile L -> (first row, rows, n-tile within its segment, segment) in
// the order above; segment s has ntiles[s] n-tiles (at most 3 segments).
template <int BM>
MOE_DEV Tile dense_tile(int L, int m_tiles, int total_ntiles, int M, int nseg, int nt0, int nt1) {
  // kNSplit column ranges, each over all m-tiles, one after the other
  int n_base = 0, n_cnt = total_ntiles;
#pragma unroll
  for (int h = 0; h < kNSplit - 1; ++h) {
    const int cnt = (total_ntiles - n_base + (kNSplit - h) - 1) / (kNSplit - h);
    if (L < m_tiles * cnt) {
      n_cnt = cnt;
      break;
    }
    L -= m_tiles * cnt;
    n_base += cnt;
    n_cnt = total_ntiles - n_base;
  }
  const int per_group = kGroupM * n_cnt;
  const int group = L / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(m_tiles - first_m, kGroupM);
  const int in_group = L - group * per_group;
  Tile t;
  t.row0 = (first_m + in_group % gm) * BM;
  t.rows = min(BM, M - t.row0);
  int nt = n_base + in_group / gm, sg = 0;
  if (nseg > 1 && nt >= nt0) {
    nt -= nt0;
    sg = 1;
    if (nseg > 2 && nt >= nt1) {
      nt -= nt1;
      sg = 2;
    }
  }
  t.nt = nt;
  t.sel = sg;
  return t;
}

template <class Pp>
struct DenseProb {
  static constexpr int PARTS = 2;
  static constexpr bool kSettleScalar = true;  // operand addresses come from kernel arguments
  template <int L>
  struct SrcT {
    const char* p[2][L];
  };
  const DenseArgs& a;
  const __attribute__((address_space(3))) float* col_lds;  // copy of the EPI_F32 segment's col_off

  MOE_DEV int total() const { return a.m_tiles * a.total_ntiles; }
  MOE_DEV int kt() const { return a.kt[0] + a.kt[1]; }
  MOE_DEV const DenseSeg& seg(int s) const { return s == 0 ? a.seg[0] : (s == 1 ? a.seg[1] : a.seg[2]); }

  MOE_DEV Tile tile(int L) const {
    return dense_tile<Pp::BM>(L, a.m_tiles, a.total_ntiles, a.M, a.nseg, a.seg[0].ntiles, a.seg[1].ntiles);
  }

  // Wave-uniform operand fields of one K part of the tile's segment, read
  // once per tile (readfirstlane is not merged across calls, so reading them
  // per slot put a chain of dependent scalar loads at every tile switch).
  struct PartSrc {
    const char *A, *gate, *up;
    int lda, ldb, N;
    bool glu;
  };

  // Start of stage row `row` (A rows first, then weight rows).
  MOE_DEV static const char* row_ptr(const Tile& t, const PartSrc& P, int row) {
    if (row < Pp::BM) {  // A row (rows past the end read row0: their results are not stored)
      const int r = row < t.rows ? row : 0;
      return P.A + (size_t)(t.row0 + r) * P.lda;
    }
    const int c = row - Pp::BM;  // weight row of tile column c (columns past N read row 0)
    int wrow;
    const char* base;
    if (P.glu) {
      wrow = t.nt * (Pp::BN / 2) + (c >> 5) * 16 + (c & 15);
      base = ((c & 31) >= 16) ? P.up : P.gate;
    } else {
      wrow = t.nt * Pp::BN + c;
      base = P.gate;
    }
    if (wrow >= P.N) wrow = 0;
    return base + (size_t)wrow * P.ldb;
  }

  template <int L>
  MOE_DEV void sources(const Tile& t, SrcT<L>& src) const {
    const int lane = threadIdx.x & 63, wave = Pp::wave_id();
    const DenseSeg& S = seg(t.sel);
    const bool glu = S.kind == EPI_GLU;
    const int N = uniform_int(S.N);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      if (a.kt[part] <= 0) {
#pragma unroll
        for (int i = 0; i < L; ++i) src.p[part][i] = nullptr;
        continue;
      }
      PartSrc P;
      P.A = uniform_ptr(a.A[part]);
      P.lda = uniform_int(a.lda_bytes[part]);
      P.gate = uniform_ptr(S.B[part]);
      P.up = glu ? uniform_ptr(S.Bu[part]) : P.gate;
      P.ldb = uniform_int(a.ldb_bytes[part]);
      P.N = N;
      P.glu = glu;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int row = Pp::slot_row(i, wave, lane);
        src.p[part][i] = row_ptr(t, P, row) + Pp::slot_chunk(row, lane) * 16;
      }
    }
  }

  template <int L>
  MOE_DEV void issue(const SrcT<L>& src, int ks, uint32_t lds) const {
    // the K part is wave-uniform: one scalar branch, not a per-slot select
    if (ks >= uniform_int(a.kt[0])) {
      const int off = (ks - uniform_int(a.kt[0])) * Pp::RB;
#pragma unroll
      for (int i = 0; i < L; ++i) lds_dma16(src.p[1][i] + off, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
    } else {
      const int off = ks * Pp::RB;
#pragma unroll
      for (int i = 0; i < L; ++i) lds_dma16(src.p[0][i] + off, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
    }
  }


  MOE_DEV void epilogue(const Tile& t, const typename Pp::Acc& acc) const {
    const DenseSeg& S = seg(t.sel);
    if (S.kind == EPI_F32)
      Pp::template epilogue<EPI_F32>(acc, t.rows, t.nt * Pp::BN, S.N, S.out, S.ldo, (size_t)t.row0,
                                     S.col_off ? col_lds : nullptr);
    else if (S.kind == EPI_GLU)
      Pp::template epilogue<EPI_GLU>(acc, t.rows, t.nt * Pp::BN, S.N, S.out, S.ldo, (size_t)t.row0, nullptr,
                                     S.keep[0], S.keep[1]);
    else
      Pp::template epilogue<EPI_STORE>(acc, t.rows, t.nt * Pp::BN, S.N, S.out, S.ldo, (size_t)t.row0, nullptr);
  }
};

// TAG only names the launch (0: the h GEMM of a forward, 1: router logits
// alone, 2: the output GEMM) so that profiles tell the dense GEMMs apart.
template <class Pp, int TAG>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_dense(const DenseArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  // Per-column offsets go through LDS: a vector load in the epilogue would
  // have to wait for every stage DMA in flight.  Copied before the first DMA.
  __shared__ float col_lds[kMaxColOff];
  for (int s = 0; s < args.nseg; ++s) {
    const DenseSeg& S = s == 0 ? args.seg[0] : (s == 1 ? args.seg[1] : args.seg[2]);
    if (S.kind == EPI_F32 && S.col_off)
      for (int i = threadIdx.x; i < S.N; i += Pp::THREADS) col_lds[i] = S.col_off[i];
  }
  __syncthreads();
  DenseProb<Pp> prob{args, (const __attribute__((address_space(3))) float*)col_lds};
  stream<Pp>(prob, smem);
}

// ---------------------------------------------------------- expert GEMMs --
// Tiles: global m-tile g (of kExpertBM rows) x n-tile; tile_info[g] =
// {first row, expert << 8 | rows in use}, written by the offsets scan; the
// m-tile count is tile_offsets[E].  Logical tile L -> m-tile L / NT, n-tile
// L % NT.
struct ExpertArgs {
  const char* A;  // z (up, gathered) or H (down, rows grouped by expert)
  int lda_bytes;
  const int32_t* gather;  // A row of grouped row r is gather[r] (NULL: r itself)
  // MXFP8 operands only: E8M0 scale rows (one byte per 32 elements of K)
  const uint8_t* sA;   // of A rows, by grouped row (already gathered)
  const uint8_t* sW;   // of W rows (gate rows for a GLU)
  const uint8_t* sWu;  // of up rows for a GLU
  int s_ld;            // scale bytes per row = K / 32
  int w_rows;          // weight rows per expert
  const char* W;   // W_g (up) or W_d (down), [E, N, K]
  const char* Wu;  // W_u (up) or nullptr
  int ldb_bytes;
  size_t w_expert_bytes;
  int N;  // output columns
  int NT;
  int kt;
  const int2* tile_info;
  const int32_t* n_mtiles;  // -> tile_offsets[E]
  void* out;
  int ldo;
  void* keep[2];  // EPI_GLU: gate / up pre-activations also stored (nullable)
};

template <class Pp, int KIND>
struct ExpertProb {
  static constexpr int PARTS = 1;
  static constexpr bool kSettleScalar = false;
  template <int L>
  struct SrcT {
    const char* p[L];
  };
  const ExpertArgs& a;

  MOE_DEV int total() const { return scalar_load(a.n_mtiles, 0) * a.NT; }
  MOE_DEV int kt() const { return a.kt; }

  MOE_DEV Tile tile(int L) const {
    const int g = L / a.NT;
    const int2 info = scalar_load2(a.tile_info, g);
    Tile t;
    t.row0 = info.x;
    t.rows = info.y & 0xFF;
    t.sel = info.y >> 8;
    t.nt = L - g * a.NT;
    return t;
  }

  // Start of stage row `row` (A rows first, then weight rows).
  MOE_DEV const char* row_ptr(const Tile& t, int row) const {
    if (row < Pp::BM)  // rows past the expert's end read its first row (results not stored)
      return uniform_ptr(a.A) + (size_t)(t.row0 + (row < t.rows ? row : 0)) * uniform_int(a.lda_bytes);
    const int c = row - Pp::BM;
    const char* gate = uniform_ptr(a.W);
    int wrow;
    const char* base;
    if (is_glu(KIND)) {
      wrow = t.nt * (Pp::BN / 2) + (c >> 5) * 16 + (c & 15);
      base = ((c & 31) >= 16) ? uniform_ptr(a.Wu) : gate;
    } else {
      wrow = t.nt * Pp::BN + c;
      base = gate;
    }
    if (wrow >= uniform_int(a.N)) wrow = 0;
    return base + (size_t)t.sel * a.w_expert_bytes + (size_t)wrow * uniform_int(a.ldb_bytes);
  }

  // Dispatch fused into the operand load: the A rows of slot group `grp`
  // (1024 / RB consecutive tile rows) are token rows gather[row0 + r] of z.
  // The indices come through scalar loads (uniform addresses), so no vector
  // load joins the DMA ring; each lane then picks the row it copies.
  MOE_DEV const char* gathered_row_ptr(const Tile& t, int grp) const {
    constexpr int R = 1024 / Pp::RB;
    const int j = (threadIdx.x & 63) / Pp::CPR;
    int src_row = 0;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int r = grp * R + q;
      const int v = scalar_load(a.gather, t.row0 + (r < t.rows ? r : 0));
      src_row = j == q ? v : src_row;
    }
    return uniform_ptr(a.A) + (size_t)src_row * uniform_int(a.lda_bytes);
  }

  template <int L>
  MOE_DEV void sources(const Tile& t, SrcT<L>& src) const {
    const int lane = threadIdx.x & 63, wave = Pp::wave_id();
    const int uwave = uniform_int(wave);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int row = Pp::slot_row(i, wave, lane);
      const int grp = i * Pp::NW + uwave;  // the slot's group of 1024 / RB rows
      const char* p = (a.gather && grp * (1024 / Pp::RB) < Pp::BM) ? gathered_row_ptr(t, grp) : row_ptr(t, row);
      src.p[i] = p + Pp::slot_chunk(row, lane) * 16;
    }
  }


  template <int L>
  MOE_DEV void issue(const SrcT<L>& src, int ks, uint32_t lds) const {
#pragma unroll
    for (int i = 0; i < L; ++i)
      lds_dma16(src.p[i] + ks * Pp::RB, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
  }

  MOE_DEV void epilogue(const Tile& t, const typename Pp::Acc& acc) const {
    Pp::template epilogue<KIND>(acc, t.rows, t.nt * Pp::BN, a.N, a.out, a.ldo, (size_t)t.row0, nullptr, a.keep[0],
                                a.keep[1]);
  }
};

template <class Pp, int KIND>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_expert(const ExpertArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  ExpertProb<Pp, KIND> prob{args};
  stream<Pp>(prob, smem);
}

// ------------------------------------ data gradients with K-major weights --
// C = A B with A row-major (K contiguous: dout, dA_cat, dY, [dA | dU]) and B
// the weights as stored, i.e. K-major ([in, out] rows of a y = x W^T layer
// read along their first index), so no transposed weight copies are made.
// K is a concatenation of up to 4 pieces: piece j covers stages [st[j],
// st[j+1]) and reads its K rows from B[j] (row stride ldb[j]); rows past
// rows[j] are read from the zero row.  Dense mode: the dense tile order over
// up to 2 output segments (each with its own pieces' sources, N and output);
// expert mode: the grouped tiles of the expert GEMMs, B advancing by
// b_expert_bytes per expert.
struct DgradSeg {
  const char* B[4];
  long long ldb[4];  // elements
  int N, ntiles, kind;
  void* out;
  int ldo;
};

struct DgradArgs {
  const char* A;
  int lda_bytes;
  int M, m_tiles, nseg, total_ntiles;  // dense mode
  DgradSeg seg[2];
  int st[5], rows[4], npiece;
  int es;
  const int2* tile_info;  // expert mode
  const int32_t* n_mtiles;
  size_t b_expert_bytes;
};

template <class Pp, bool EXPERT>
struct DgradProb {
  static constexpr int PARTS = 1;
  static constexpr bool kSettleScalar = false;
  static constexpr int LA = Pp::LA, KR = Pp::KR;
  template <int L>
  struct SrcT {
    const char* pa[LA];       // A chunk addresses at the first stage
    uint32_t cb[L - LA];      // B chunk byte offsets within a K row
    int sel;                  // the tile's segment (dense) or expert (wave-uniform)
  };
  const DgradArgs& a;

  MOE_DEV int total() const {
    if constexpr (EXPERT) return scalar_load(a.n_mtiles, 0) * a.seg[0].ntiles;
    else return a.m_tiles * a.total_ntiles;
  }
  MOE_DEV int kt() const { return a.st[a.npiece]; }
  MOE_DEV Tile tile(int L) const {
    if constexpr (EXPERT) {
      const int NT = a.seg[0].ntiles, g = L / NT;
      const int2 info = scalar_load2(a.tile_info, g);
      Tile t;
      t.row0 = info.x;
      t.rows = info.y & 0xFF;
      t.sel = info.y >> 8;
      t.nt = L - g * NT;
      return t;
    } else {
      return dense_tile<Pp::BM>(L, a.m_tiles, a.total_ntiles, a.M, a.nseg, a.seg[0].ntiles, 0);
    }
  }
  MOE_DEV const DgradSeg& seg(const Tile& t) const {
    if constexpr (EXPERT) return a.seg[0];
    else return t.sel == 0 ? a.seg[0] : a.seg[1];
  }
  template <int L>
  MOE_DEV void sources(const Tile& t, SrcT<L>& src) const {
    const int lane = threadIdx.x & 63, wave = Pp::wave_id(), uwave = uniform_int(wave);
    const DgradSeg& S = seg(t);
    const size_t es = uniform_int(a.es);
    const int lda = uniform_int(a.lda_bytes), N = uniform_int(S.N);
#pragma unroll
    for (int i = 0; i < LA; ++i) {  // A rows past the tile's end read its first row (not stored)
      const int row = Pp::slot_row(i, wave, lane);
      src.pa[i] = uniform_ptr(a.A) + (size_t)(t.row0 + (row < t.rows ? row : 0)) * lda + Pp::slot_chunk(row, lane) * 16;
    }
#pragma unroll
    for (int i = LA; i < L; ++i) {
      const int row = Pp::template km_slot_row<Pp::PB>((i - LA) * Pp::NW + uwave, lane);
      int col = t.nt * Pp::BN + Pp::template km_slot_colbyte<Pp::PB>(row, lane) / (int)es;
      if (col >= N) col = 0;
      src.cb[i - LA] = (uint32_t)(col * es);
    }
    src.sel = t.sel;
  }
  template <int L>
  MOE_DEV void issue(const SrcT<L>& src, int ks, uint32_t lds) const {
    const int lane = threadIdx.x & 63, uwave = uniform_int(Pp::wave_id());
#pragma unroll
    for (int i = 0; i < LA; ++i)
      lds_dma16(src.pa[i] + ks * Pp::RB, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
    // the stage's piece and its source, from the kernel arguments (wave-uniform)
    int j = 0;
#pragma unroll
    for (int q = 1; q < 4; ++q) j = (q < a.npiece && ks >= a.st[q]) ? q : j;
    j = uniform_int(j);
    const int sel = uniform_int(src.sel);
    const DgradSeg& S = EXPERT || sel == 0 ? a.seg[0] : a.seg[1];
    const char* B = uniform_ptr(S.B[j] + (EXPERT ? (size_t)sel * a.b_expert_bytes : 0));
    const size_t ldb = (size_t)uniform_ll(S.ldb[j]) * uniform_int(a.es);
    const int rows = uniform_int(a.rows[j]);
    const int kr0 = uniform_int((ks - a.st[j]) * KR);
    const char* zero = reinterpret_cast<const char*>(g_zero_row) + (lane << 4);
#pragma unroll
    for (int i = LA; i < L; ++i) {
      const int kr = kr0 + Pp::template km_slot_row<Pp::PB>((i - LA) * Pp::NW + uwave, lane);
      const char* q = kr < rows ? B + (size_t)kr * ldb + src.cb[i - LA] : zero;
      lds_dma16(q, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
    }
  }
  MOE_DEV void epilogue(const Tile& t, const typename Pp::Acc& acc) const {
    const DgradSeg& S = seg(t);
    if (!EXPERT && S.kind == EPI_F32)
      Pp::template epilogue<EPI_F32>(acc, t.rows, t.nt * Pp::BN, S.N, S.out, S.ldo, (size_t)t.row0, nullptr);
    else
      Pp::template epilogue<EPI_STORE>(acc, t.rows, t.nt * Pp::BN, S.N, S.out, S.ldo, (size_t)t.row0, nullptr);
  }
};

// TAG names the launch for profiles (4: dout products, 5: dh, 8: expert dH,
// 9: expert dX).
template <class Pp, bool EXPERT, int TAG>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_dgrad(const DgradArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  DgradProb<Pp, EXPERT> prob{args};
  stream<Pp>(prob, smem);
}

// The persistent stream for tiles whose K length varies (kt_of(tile) >= 1
// stages): the issue and the compute cursors each track their own tile's
// length; otherwise as stream().
template <class Pp, class Prob>
MOE_DEV void stream_var(const Prob& prob, char* smem) {
  const int G = gridDim.x, b = blockIdx.x;
  const int x = b & 7, q = b >> 3, Gx = G >> 3;
  const int total_tiles = prob.total();
  const int per = (total_tiles + 7) >> 3;
  const int lo = x * per, hi = min(total_tiles, lo + per);
  const int span = hi - lo - q;
  const int my_n = span > 0 ? (span + Gx - 1) / Gx : 0;
  if (my_n <= 0) return;
  const uint32_t lds0 = lds_addr(smem) + Pp::wave_id() * 1024;

  typename Prob::template SrcT<Pp::L> src;
  int iss_j = 0, iss_ks = 0, issued = 0;
  Tile it = prob.tile(lo + q);
  int iss_kt = prob.kt_of(it);
  prob.sources(it, src);
  auto issue = [&]() {
    const uint32_t base = lds0 + (uint32_t)((issued % Pp::NS) * Pp::STAGE);
    prob.issue(src, iss_ks, base);
    ++issued;
    if (++iss_ks == iss_kt) {
      iss_ks = 0;
      if (++iss_j < my_n) {
        it = prob.tile(lo + q + iss_j * Gx);
        iss_kt = prob.kt_of(it);
        prob.sources(it, src);
      }
    }
  };
  for (int s = 0; s < Pp::NS - 1; ++s)
    if (iss_j < my_n) issue();

  typename Pp::Acc acc;
  Pp::zero(acc);
  int cj = 0, cks = 0;
  Tile ct = prob.tile(lo + q);
  int ckt = prob.kt_of(ct);
  for (int g = 0; cj < my_n; ++g) {
    Pp::wait_stage(issued - g - 1);
    block_barrier();
    if (iss_j < my_n) issue();
    Pp::compute(smem + (g % Pp::NS) * Pp::STAGE, acc);
    if (++cks == ckt) {
      prob.epilogue(ct, acc);
      Pp::zero(acc);
      cks = 0;
      if (++cj < my_n) {
        ct = prob.tile(lo + q + cj * Gx);
        ckt = prob.kt_of(ct);
      }
    }
  }
}

// ------------------------------- weight gradients from token-major operands --
// C_e = A_e^T B_e for every segment e of the token (K) axis, with A and B
// stored token-major (row k holds that token's M or N values), so neither is
// transposed in memory: both enter the MFMA through K-major LDS regions.
// Segment e covers rows [koff[e], koff[e+1]) (koff == nullptr: [e kstep,
// (e+1) kstep)), cut at kend; rows past the segment's end, up to its last
// whole stage, are read from a zero row.  B's columns n < nsplit come from
// B[0], the rest from B[1] (two operands side by side, e.g. [G | y_lat]);
// with `gather`, B's row k is row gather[k] (the dispatch permutation).
// C_e [M, N] fp32 at out + e M N.
struct WgradKmArgs {
  const char* A;
  const char* B[2];
  long long lda, ldb[2];  // row strides, elements
  const int32_t* koff;
  const int32_t* gather;
  int kstep, kend, ngather, nsplit;
  int es, M, N, MT, NT, E;
  float* out;
};

template <class Pp>
struct WgradKmProb {
  static constexpr int PARTS = 1;
  static constexpr int LA = Pp::LA, KR = Pp::KR;
  template <int L>
  struct SrcT {
    const char* p[L];   // chunk address at the first stage (gathered B: at row 0)
    uint32_t stride[L]; // bytes per stage (gathered B: per row)
    int k0, n;          // the segment's first row and row count (wave-uniform)
  };
  const WgradKmArgs& a;

  MOE_DEV int total() const { return a.E * a.MT * a.NT; }
  MOE_DEV Tile tile(int L) const {
    const int per = a.MT * a.NT;
    const int e = L / per, r = L - e * per;
    const int mt = r / a.NT;
    Tile t;
    t.row0 = mt * Pp::BM;
    t.rows = min(Pp::BM, a.M - t.row0);
    t.nt = r - mt * a.NT;
    t.sel = e;
    return t;
  }
  MOE_DEV int2 seg(const Tile& t) const {  // first row, row count
    const int kend = uniform_int(a.kend);
    int k0, k1;
    if (a.koff) {
      k0 = scalar_load(a.koff, t.sel);
      k1 = scalar_load(a.koff, t.sel + 1);
    } else {
      k0 = t.sel * uniform_int(a.kstep);
      k1 = k0 + uniform_int(a.kstep);
    }
    k1 = min(k1, kend);
    return make_int2(k0, max(0, k1 - k0));
  }
  MOE_DEV int kt_of(const Tile& t) const { return max(1, (seg(t).y + KR - 1) / KR); }
  template <int L>
  MOE_DEV void sources(const Tile& t, SrcT<L>& src) const {
    const int lane = threadIdx.x & 63, wave = uniform_int(Pp::wave_id());
    const int2 sg = seg(t);
    src.k0 = sg.x;
    src.n = sg.y;
    const size_t es = uniform_int(a.es);
    const int M = uniform_int(a.M), N = uniform_int(a.N), nsplit = uniform_int(a.nsplit);
    const bool gather = a.gather != nullptr;
    const size_t lda = (size_t)uniform_ll(a.lda), ldb0 = (size_t)uniform_ll(a.ldb[0]),
                 ldb1 = (size_t)uniform_ll(a.ldb[1]);
    const char *A = uniform_ptr(a.A), *B0 = uniform_ptr(a.B[0]), *B1 = uniform_ptr(a.B[1]);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int si = i * Pp::NW + wave;
      if (i < LA) {
        const int row = Pp::template km_slot_row<Pp::PA>(si, lane);
        int col = t.row0 + Pp::template km_slot_colbyte<Pp::PA>(row, lane) / (int)es;
        if (col >= M) col = 0;
        src.p[i] = A + ((size_t)(sg.x + row) * lda + col) * es;
        src.stride[i] = (uint32_t)(KR * lda * es);
      } else {
        const int row = Pp::template km_slot_row<Pp::PB>(si - LA * Pp::NW, lane);
        int col = t.nt * Pp::BN + Pp::template km_slot_colbyte<Pp::PB>(row, lane) / (int)es;
        if (col >= N) col = 0;
        const bool second = col >= nsplit;
        const char* base = second ? B1 : B0;
        const size_t ld = second ? ldb1 : ldb0;
        const size_t c = (size_t)(second ? col - nsplit : col);
        if (gather) {
          src.p[i] = base + c * es;
          src.stride[i] = (uint32_t)(ld * es);
        } else {
          src.p[i] = base + ((size_t)(sg.x + row) * ld + c) * es;
          src.stride[i] = (uint32_t)(KR * ld * es);
        }
      }
    }
  }
  template <int L>
  MOE_DEV void issue(const SrcT<L>& src, int ks, uint32_t lds) const {
    const int lane = threadIdx.x & 63, wave = uniform_int(Pp::wave_id());
    const char* zero = reinterpret_cast<const char*>(g_zero_row) + (lane << 4);
    const bool gather = a.gather != nullptr;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int si = i * Pp::NW + wave;
      const char* q;
      int row;
      if (i < LA) {
        row = Pp::template km_slot_row<Pp::PA>(si, lane);
        q = src.p[i] + (size_t)ks * src.stride[i];
      } else {
        constexpr int RPS = 1024 / Pp::PB, LPR = Pp::PB / 16;  // rows per slot, lanes per row
        const int ls = si - LA * Pp::NW;
        row = Pp::template km_slot_row<Pp::PB>(ls, lane);
        if (gather) {  // the slot's RPS rows: scalar loads of their source rows
          const int first = uniform_int(src.k0 + ks * KR + ls * RPS), last = uniform_int(a.ngather) - 1;
          int gi = 0;
#pragma unroll
          for (int j = 0; j < RPS; ++j) {
            const int v = scalar_load(a.gather, min(first + j, last));
            gi = lane / LPR == j ? v : gi;
          }
          q = src.p[i] + (size_t)gi * src.stride[i];
        } else {
          q = src.p[i] + (size_t)ks * src.stride[i];
        }
      }
      if (ks * KR + row >= src.n) q = zero;
      lds_dma16(q, __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
    }
  }
  MOE_DEV void epilogue(const Tile& t, const typename Pp::Acc& acc) const {
    Pp::template epilogue<EPI_F32>(acc, t.rows, t.nt * Pp::BN, a.N, a.out + (size_t)t.sel * a.M * a.N, a.N,
                                   (size_t)t.row0, nullptr);
  }
};

template <class Pp>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_wgrad_km(const WgradKmArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  WgradKmProb<Pp> prob{args};
  stream_var<Pp>(prob, smem);
}

// ------------------------------------------------ MXFP8 expert GEMMs --
// Operands are FP8 E4M3 bytes with one E8M0 scale per 32 elements along K
// (OCP microscaling); one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 block
// and 128-byte stage.  Its operand layout (measured on gfx950): lane (i, g =
// lane / 16) holds K bytes [16g, 16g+16) and [64+16g, 64+16g+16) of row i of
// the window, i.e. logical 16-byte chunks g and 4+g of the LDS row; the scale
// it supplies (byte 0 of the operand) is that of row i's block g of 32.  The
// DMA ring, LDS layout and epilogues are those of the bf16 expert GEMM.
typedef int v8i_t __attribute__((ext_vector_type(8)));

// Byte g (the lane's 32-element block) of the current stage's scale word,
// which is always w[0]: the words then move down one place for the next
// stage (the tile's stages run in order from 0 and the next tile reloads
// them).  Indexing the words by the stage number instead made the compiler
// branch on it between MFMAs, or keep the words in scratch memory.
MOE_DEV int mx_take(uint32_t (&w)[4], int g) {
  const int v = (int)((w[0] >> (8 * g)) & 0xFFu);
  w[0] = w[1];
  w[1] = w[2];
  w[2] = w[3];
  return v;
}

template <class Pp>
MOE_DEV void mx_compute(const char* cur, typename Pp::Acc& acc, uint32_t (&sa)[Pp::MI][4],
                        uint32_t (&sb)[Pp::NI][4]) {
  const int lane = threadIdx.x & 63, wave = Pp::wave_id();
  const int wm = wave / Pp::WN, wn = wave % Pp::WN, g = lane >> 4;
  v8i_t af[Pp::MI], wf[Pp::NI];
#pragma unroll
  for (int ni = 0; ni < Pp::NI; ++ni) {
    const int row = Pp::BM + wn * Pp::WTN + ni * 16 + (lane & 15);
    const uint4 lo = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, g));
    const uint4 hi = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, 4 + g));
    wf[ni] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi) {
    const int row = wm * Pp::WTM + mi * 16 + (lane & 15);
    const uint4 lo = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, g));
    const uint4 hi = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, 4 + g));
    af[mi] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // the stage's scale byte of every row and weight fragment, taken once
  // before the MFMAs
  int scA[Pp::MI], scB[Pp::NI];
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi) scA[mi] = mx_take(sa[mi], g);
#pragma unroll
  for (int ni = 0; ni < Pp::NI; ++ni) scB[ni] = mx_take(sb[ni], g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < Pp::NI; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[ni], af[mi], acc[mi][ni], 0, 0, 0, scB[ni],
                                                                     0, scA[mi]);
}

template <class Pp, int KIND>
struct ExpertMxProb : ExpertProb<Pp, KIND> {
  using ExpertProb<Pp, KIND>::a;
  // The scale words (4 bytes = the 4 blocks of one 128-byte stage; K <= 512)
  // of the lane's A rows and weight rows for tile t.  Vector loads: the
  // caller consumes them before its next DMA issue.
  MOE_DEV void load_scales(const Tile& t, uint32_t (&sa)[Pp::MI][4], uint32_t (&sb)[Pp::NI][4]) const {
    const int lane = threadIdx.x & 63, wave = Pp::wave_id();
    const int wm = wave / Pp::WN, wn = wave % Pp::WN;
    const int sld = uniform_int(a.s_ld), nd = sld / 4;
#pragma unroll
    for (int mi = 0; mi < Pp::MI; ++mi) {
      const int lr = wm * Pp::WTM + mi * 16 + (lane & 15);
      const int gr = t.row0 + (lr < t.rows ? lr : 0);
      const uint32_t* p = reinterpret_cast<const uint32_t*>(a.sA + (size_t)gr * sld);
#pragma unroll
      for (int q = 0; q < 4; ++q) sa[mi][q] = q < nd ? p[q] : 0u;
    }
#pragma unroll
    for (int ni = 0; ni < Pp::NI; ++ni) {
      const int c = wn * Pp::WTN + ni * 16 + (lane & 15);
      int wrow;
      const uint8_t* base;
      if (is_glu(KIND)) {
        wrow = t.nt * (Pp::BN / 2) + (c >> 5) * 16 + (c & 15);
        base = (c & 31) >= 16 ? a.sWu : a.sW;
      } else {
        wrow = t.nt * Pp::BN + c;
        base = a.sW;
      }
      if (wrow >= a.N) wrow = 0;
      const uint32_t* p =
          reinterpret_cast<const uint32_t*>(base + ((size_t)t.sel * a.w_rows + wrow) * (size_t)sld);
#pragma unroll
      for (int q = 0; q < 4; ++q) sb[ni][q] = q < nd ? p[q] : 0u;
    }
  }
};

// MXFP4 weights (4-bit E2M1 elements, two per byte, low nibble first, one
// E8M0 scale per 32 along K) against MXFP8 activations.  The FP4 operand of
// v_mfma_scale_f32_16x16x128_f8f6f4 (cbsz = 4, measured on gfx950): lane (i,
// g = lane / 16) holds K elements [32g, 32g+32) of row i as 16 contiguous
// bytes, and its scale byte scales exactly those; the upper half of the
// 8-register operand is not read.  A stage covers 128 K values: activation
// rows of 128 bytes as in the MXFP8 GEMM, weight rows of 64 bytes (16-byte
// chunk j of weight row c at position j ^ (c / 2) % 4).
template <int BM_, int BN_, int WM_, int WN_, int NS_, int BPC_>
struct Mx4Pipe : Pipe<BM_, BN_, WM_, WN_, NS_, 128, BPC_, true> {
  using Base = Pipe<BM_, BN_, WM_, WN_, NS_, 128, BPC_, true>;
  static constexpr int RBW = 64;
  static constexpr int STAGE = Base::A_BYTES + Base::BN * RBW;
  static constexpr int LDS = Base::NS * STAGE;
  static constexpr int L = STAGE / 1024 / Base::NW;
  static constexpr int LA = Base::A_BYTES / (1024 * Base::NW);
  static_assert(STAGE % (1024 * Base::NW) == 0 && Base::A_BYTES % (1024 * Base::NW) == 0, "whole DMA slots");
  static_assert(LDS * Base::BPC <= 160 * 1024, "LDS per CU");
  MOE_DEV static int w_off(int c, int j) { return Base::A_BYTES + c * RBW + ((j ^ ((c >> 1) & 3)) << 4); }
  MOE_DEV static void wait_stage(int after) {
    if (after <= 0) wait_vmcnt<0>();
    else if (after == 1) wait_vmcnt<L>();
    else wait_vmcnt<2 * L>();
  }
};

template <class Pp>
MOE_DEV void mx4_compute(const char* cur, typename Pp::Acc& acc, uint32_t (&sa)[Pp::MI][4],
                         uint32_t (&sb)[Pp::NI][4]) {
  const int lane = threadIdx.x & 63, wave = Pp::wave_id();
  const int wm = wave / Pp::WN, wn = wave % Pp::WN, g = lane >> 4;
  v8i_t af[Pp::MI], wf[Pp::NI];
#pragma unroll
  for (int ni = 0; ni < Pp::NI; ++ni) {
    const uint4 w = *reinterpret_cast<const uint4*>(cur + Pp::w_off(wn * Pp::WTN + ni * 16 + (lane & 15), g));
    wf[ni] = v8i_t{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi) {
    const int row = wm * Pp::WTM + mi * 16 + (lane & 15);
    const uint4 lo = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, g));
    const uint4 hi = *reinterpret_cast<const uint4*>(cur + Pp::lds_off(row, 4 + g));
    af[mi] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // the stage's scale byte of every row and weight fragment, taken once
  // before the MFMAs
  int scA[Pp::MI], scB[Pp::NI];
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi) scA[mi] = mx_take(sa[mi], g);
#pragma unroll
  for (int ni = 0; ni < Pp::NI; ++ni) scB[ni] = mx_take(sb[ni], g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 0; mi < Pp::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < Pp::NI; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[ni], af[mi], acc[mi][ni], 4, 0, 0, scB[ni],
                                                                     0, scA[mi]);
}

template <class Pp, int KIND>
struct ExpertMx4Prob : ExpertMxProb<Pp, KIND> {
  using ExpertMxProb<Pp, KIND>::a;
  template <int L>
  using SrcT = typename ExpertProb<Pp, KIND>::template SrcT<L>;
  template <int L>
  MOE_DEV void sources(const Tile& t, SrcT<L>& src) const {
    const int lane = threadIdx.x & 63, wave = Pp::wave_id(), uwave = uniform_int(wave);
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < Pp::LA) {  // activation rows: as the MXFP8 GEMM
        const int row = Pp::slot_row(i, wave, lane);
        const int grp = i * Pp::NW + uwave;
        const char* p = a.gather ? this->gathered_row_ptr(t, grp) : this->row_ptr(t, row);
        src.p[i] = p + Pp::slot_chunk(row, lane) * 16;
      } else {  // weight rows of 64 bytes: 16 per slot, 4 lanes each
        const int c = ((i - Pp::LA) * Pp::NW + wave) * 16 + lane / 4;
        src.p[i] = this->row_ptr(t, Pp::BM + c) + (((lane & 3) ^ ((c >> 1) & 3)) << 4);
      }
    }
  }
  template <int L>
  MOE_DEV void issue(const SrcT<L>& src, int ks, uint32_t lds) const {
#pragma unroll
    for (int i = 0; i < L; ++i)
      lds_dma16(src.p[i] + ks * (i < Pp::LA ? Pp::RB : Pp::RBW),
                __builtin_amdgcn_readfirstlane(lds + i * Pp::NW * 1024));
  }
};

// The persistent stream of the block-scaled expert GEMMs (W4: MXFP4 weights).
template <class Pp, class Prob, bool W4>
MOE_DEV void expert_mx_stream(const ExpertArgs& args, char* smem) {
  Prob prob{args};
  const int G = gridDim.x, b = blockIdx.x;
  const int x = b & 7, q = b >> 3, Gx = G >> 3;
  const int total_tiles = prob.total();
  const int per = (total_tiles + 7) >> 3;
  const int lo = x * per, hi = min(total_tiles, lo + per);
  const int span = hi - lo - q;
  const int my_n = span > 0 ? (span + Gx - 1) / Gx : 0;
  if (my_n <= 0) return;
  const int KT = prob.kt();
  const int total = my_n * KT;
  const uint32_t lds0 = lds_addr(smem) + Pp::wave_id() * 1024;
  typename Prob::template SrcT<Pp::L> src;
  int iss_j = 0, iss_ks = 0, issued = 0;
  prob.sources(prob.tile(lo + q), src);
  auto issue = [&]() {
    const uint32_t base = lds0 + (uint32_t)((issued % Pp::NS) * Pp::STAGE);
    prob.issue(src, iss_ks, base);
    ++issued;
    if (++iss_ks == KT) {
      iss_ks = 0;
      if (++iss_j < my_n) prob.sources(prob.tile(lo + q + iss_j * Gx), src);
    }
  };
  uint32_t sa[Pp::MI][4], sb[Pp::NI][4];
  Tile ct = prob.tile(lo + q);
  prob.load_scales(ct, sa, sb);
  for (int s0 = 0; s0 < Pp::NS - 1; ++s0)
    if (issued < total) issue();
  typename Pp::Acc acc;
  Pp::zero(acc);
  int cj = 0, cks = 0;
  for (int g = 0; g < total; ++g) {
    Pp::wait_stage(issued - g - 1);
    block_barrier();
    // use the scale words here: the compiler's wait for their loads then
    // comes before the next DMA issue instead of draining it
#pragma unroll
    for (int i = 0; i < Pp::MI; ++i) asm volatile("" ::"v"(sa[i][0]), "v"(sa[i][1]), "v"(sa[i][2]), "v"(sa[i][3]));
#pragma unroll
    for (int i = 0; i < Pp::NI; ++i) asm volatile("" ::"v"(sb[i][0]), "v"(sb[i][1]), "v"(sb[i][2]), "v"(sb[i][3]));
    if (issued < total) issue();
    if constexpr (W4) mx4_compute<Pp>(smem + (g % Pp::NS) * Pp::STAGE, acc, sa, sb);
    else mx_compute<Pp>(smem + (g % Pp::NS) * Pp::STAGE, acc, sa, sb);
    if (++cks == KT) {
      prob.epilogue(ct, acc);
      Pp::zero(acc);
      cks = 0;
      if (++cj < my_n) {
        ct = prob.tile(lo + q + cj * Gx);
        prob.load_scales(ct, sa, sb);
      }
    }
  }
}

template <class Pp, int KIND>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_expert_mx(const ExpertArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  expert_mx_stream<Pp, ExpertMxProb<Pp, KIND>, false>(args, smem);
}

template <class Pp, int KIND>
__global__ __launch_bounds__(Pp::THREADS, Pp::BPC * Pp::NW / 4) void k_gemm_expert_mx4(const ExpertArgs args) {
  __shared__ __attribute__((aligned(1024))) char smem[Pp::LDS];
  expert_mx_stream<Pp, ExpertMx4Prob<Pp, KIND>, true>(args, smem);
}

// MXFP8 quantisation of rows: each block of 32 consecutive elements gets the
// scale 2^(floor(log2 amax) - 8) (E8M0 byte, clamped to [0, 254], 0 for an
// all-zero block) and E4M3 elements, round to nearest even, saturating at 448.
// W4: MXFP4 instead (scale 2^(floor(log2 amax) - 2), E2M1 elements, two per
// byte, low nibble first; dst rows of K / 2 bytes).
template <bool W4>
__global__ __launch_bounds__(256) void k_mx_quant(const uint16_t* __restrict__ src, long long rows, int K,
                                                  long long ld_src, uint8_t* __restrict__ dst,
                                                  uint8_t* __restrict__ scales) {
  const int nb = K / 32;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nb) return;
  const long long r = i / nb;
  const int bk = (int)(i - r * nb);
  const uint4* p = reinterpret_cast<const uint4*>(src + r * ld_src + (long long)bk * 32);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = p[q];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * q + 2 * h] = bf16_bits_to_f32(ww[h] & 0xFFFFu);
      v[8 * q + 2 * h + 1] = bf16_bits_to_f32(ww[h] >> 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  int byte = 0;
  if (amax > 0.f) {
    int e;
    (void)frexpf(amax, &e);
    byte = min(254, max(0, e - 1 - (W4 ? 2 : 8) + 127));
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = ldexpf(v[j], 127 - byte);
  if constexpr (W4) {
    uint32_t o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = e2m1x8(v + 8 * w);
    *reinterpret_cast<uint4*>(dst + r * (K / 2) + (long long)bk * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    scales[r * nb + bk] = (uint8_t)byte;
    return;
  }
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) o[w] = e4m3x4(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3]);
  uint4* d = reinterpret_cast<uint4*>(dst + r * K + (long long)bk * 32);
  d[0] = make_uint4(o[0], o[1], o[2], o[3]);
  d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  scales[r * nb + bk] = (uint8_t)byte;
}

// Tile shapes and pipeline depths: BM, BN, WM, WN, NS, RB, BPC.
#ifndef MOE_DENSE_CFG
#define MOE_DENSE_CFG 128, 128, 2, 2, 2, 128, 2
#endif
#ifndef MOE_EXPERT_CFG
#define MOE_EXPERT_CFG kExpertBM, 256, 1, 4, 2, 128, 2
#endif
template <bool BF16>
using DensePipe = Pipe<MOE_DENSE_CFG, BF16>;
template <bool BF16>
using ExpertPipe = Pipe<MOE_EXPERT_CFG, BF16>;
// bf16/fp32 expert down-projection over the kExpertBM2-row tile table: 4
// wavefronts of 64x128, 3 stages of 64-byte rows, 2 blocks per CU.
#ifndef MOE_EXPERT_DOWN_CFG
#define MOE_EXPERT_DOWN_CFG kExpertBM2, 256, 2, 2, 3, 64, 2
#endif
template <bool BF16>
using ExpertDownPipe = Pipe<MOE_EXPERT_DOWN_CFG, BF16>;
// expert_up over the kExpertBM2-row table, for many rows per expert
template <bool BF16>
using ExpertUpPipe2 = Pipe<MOE_EXPERT_DOWN_CFG, BF16>;
#ifndef MOE_WGRAD_CFG
#define MOE_WGRAD_CFG MOE_DENSE_CFG
#endif
template <bool BF16>
using WgradKmPipe = Pipe<MOE_WGRAD_CFG, BF16, 3>;
template <bool BF16>
using DgradPipe = Pipe<MOE_DENSE_CFG, BF16, 2>;
template <bool BF16>
using DgradExpertPipe = Pipe<MOE_EXPERT_CFG, BF16, 2>;
// MXFP8 experts: one 128-element K step (128 bytes) per stage
#ifndef MOE_EXPERT_MX_CFG
#define MOE_EXPERT_MX_CFG kExpertBM, 256, 1, 4, 2, 128, 2
#endif
using ExpertMxPipe = Pipe<MOE_EXPERT_MX_CFG, true>;
constexpr int kCUs = 256;

}  // namespace

static int esz(const Dims& D) { return D.bf16 ? 2 : 4; }

// Persistent grid: at most bpc blocks per CU, a multiple of 8.
static int persistent_grid(long long tiles, int bpc) {
  long long g = (long long)kCUs * bpc;
  if (tiles < g) g = (tiles + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

template <bool BF16, int TAG>
static hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  using P = DensePipe<BF16>;
  const long long tiles = (long long)a.m_tiles * a.total_ntiles;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_dense<P, TAG>), dim3(persistent_grid(tiles, P::BPC)), dim3(P::THREADS), 0, s,
                     a);
  return hipGetLastError();
}

template <int TAG>
static hipError_t launch_dense_any(const Dims& D, const DenseArgs& a, hipStream_t s) {
  return D.bf16 ? launch_dense<true, TAG>(a, s) : launch_dense<false, TAG>(a, s);
}

// One K pass over h for the given segments (in this order: router logits,
// shared GLU, latent z); a NULL output drops its segment.
template <int TAG>
static hipError_t launch_gemm_hsegs(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                                    const void* W_sg, const void* W_su, const void* W_dn, float* logits, void* G,
                                    void* z, hipStream_t s, void* P = nullptr, void* Q = nullptr) {
  constexpr int BM = DensePipe<true>::BM, BN = DensePipe<true>::BN, RB = DensePipe<true>::RB;
  const int es = esz(D);
  DenseArgs a{};
  a.A[0] = static_cast<const char*>(h);
  a.lda_bytes[0] = D.d * es;
  a.ldb_bytes[0] = D.d * es;
  a.kt[0] = D.d * es / RB;
  a.kt[1] = 0;
  a.M = T;
  a.m_tiles = (T + BM - 1) / BM;
  int ns = 0;
  if (logits) {  // router logits, fp32
    if (logit_offset && D.E > kMaxColOff) return hipErrorInvalidValue;
    DenseSeg& g = a.seg[ns++];
    g.B[0] = static_cast<const char*>(W_r);
    g.N = D.E;
    g.ntiles = (D.E + BN - 1) / BN;
    g.kind = EPI_F32;
    g.out = logits;
    g.ldo = D.E;
    g.col_off = logit_offset;
  }
  if (D.f_s > 0 && G) {  // shared GLU hidden
    DenseSeg& g = a.seg[ns++];
    g.B[0] = static_cast<const char*>(W_sg);
    g.Bu[0] = static_cast<const char*>(W_su);
    g.N = D.f_s;
    g.ntiles = (2 * D.f_s + BN - 1) / BN;
    g.kind = EPI_GLU;
    g.out = G;
    g.ldo = D.f_s;
    g.keep[0] = P;
    g.keep[1] = Q;
  }
  if (z) {  // latent z
    DenseSeg& g = a.seg[ns++];
    g.B[0] = static_cast<const char*>(W_dn);
    g.N = D.l;
    g.ntiles = (D.l + BN - 1) / BN;
    g.kind = EPI_STORE;
    g.out = z;
    g.ldo = D.l;
  }
  if (ns == 0) return hipSuccess;
  a.nseg = ns;
  a.total_ntiles = 0;
  for (int i = 0; i < ns; ++i) a.total_ntiles += a.seg[i].ntiles;
  return launch_dense_any<TAG>(D, a, s);
}

hipError_t launch_gemm_h(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                         const void* W_sg, const void* W_su, const void* W_dn, float* logits, void* G, void* z,
                         hipStream_t s, void* P, void* Q) {
  if ((P == nullptr) != (Q == nullptr)) return hipErrorInvalidValue;
  return launch_gemm_hsegs<0>(D, h, T, W_r, logit_offset, W_sg, W_su, W_dn, logits, G, z, s, P, Q);
}

hipError_t launch_gemm_rz(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                          float* logits, hipStream_t s) {
  return launch_gemm_hsegs<1>(D, h, T, W_r, logit_offset, nullptr, nullptr, nullptr, logits, nullptr, nullptr, s);
}

hipError_t launch_gemm_out(const Dims& D, const void* G, const void* y_lat, int T, const void* W_sd,
                           const void* W_up, void* out, hipStream_t s) {
  constexpr int BM = DensePipe<true>::BM, BN = DensePipe<true>::BN, RB = DensePipe<true>::RB;
  const int es = esz(D);
  DenseArgs a{};
  int p = 0;
  if (D.f_s > 0) {
    a.A[p] = static_cast<const char*>(G);
    a.lda_bytes[p] = D.f_s * es;
    a.ldb_bytes[p] = D.f_s * es;
    a.kt[p] = D.f_s * es / RB;
    a.seg[0].B[p] = static_cast<const char*>(W_sd);
    ++p;
  }
  a.A[p] = static_cast<const char*>(y_lat);
  a.lda_bytes[p] = D.l * es;
  a.ldb_bytes[p] = D.l * es;
  a.kt[p] = D.l * es / RB;
  a.seg[0].B[p] = static_cast<const char*>(W_up);
  a.M = T;
  a.m_tiles = (T + BM - 1) / BM;
  a.seg[0].N = D.d;
  a.seg[0].ntiles = (D.d + BN - 1) / BN;
  a.seg[0].kind = EPI_STORE;
  a.seg[0].out = out;
  a.seg[0].ldo = D.d;
  a.nseg = 1;
  a.total_ntiles = a.seg[0].ntiles;
  return launch_dense_any<2>(D, a, s);
}

int expert_max_mtiles(int T, int k, int E, int bm) {
  // sum_e ceil(n_e / BM) <= ceil(T*k / BM) + E (at most one partial tile per expert)
  return (int)(((long long)T * k + bm - 1) / bm + E);
}

template <int KIND, template <bool> class PipeT = ExpertPipe>
static hipError_t launch_expert(const Dims& D, const ExpertArgs& a, int T, hipStream_t s) {
  static_assert(PipeT<true>::BM == PipeT<false>::BM, "one tile table per pipe");
  const long long tiles = (long long)expert_max_mtiles(T, D.k, D.E, PipeT<true>::BM) * a.NT;
  if (tiles == 0) return hipSuccess;
  const int grid = persistent_grid(tiles, PipeT<true>::BPC);
  if (D.bf16)
    hipLaunchKernelGGL((k_gemm_expert<PipeT<true>, KIND>), dim3(grid), dim3(PipeT<true>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_expert<PipeT<false>, KIND>), dim3(grid), dim3(PipeT<false>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expert_up(const Dims& D, const void* z, const int32_t* perm_src, const int2* tile_info,
                            const int32_t* n_mtiles, int T, const void* W_g, const void* W_u, void* H, hipStream_t s,
                            void* A, void* U, bool tall) {
  if ((A == nullptr) != (U == nullptr)) return hipErrorInvalidValue;
  static_assert(ExpertUpPipe2<true>::BN == ExpertPipe<true>::BN, "one column tiling for both tile heights");
  constexpr int BN = ExpertPipe<true>::BN;
  const int RB = tall ? ExpertUpPipe2<true>::RB : ExpertPipe<true>::RB;  // the launched pipeline's stage rows
  const int es = esz(D);
  ExpertArgs a{};
  a.A = static_cast<const char*>(z);
  a.lda_bytes = D.l * es;
  a.gather = perm_src;
  a.W = static_cast<const char*>(W_g);
  a.Wu = static_cast<const char*>(W_u);
  a.ldb_bytes = D.l * es;
  a.w_expert_bytes = (size_t)D.f * D.l * es;
  a.N = D.f;
  a.NT = (2 * D.f + BN - 1) / BN;
  a.kt = D.l * es / RB;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.keep[0] = A;
  a.keep[1] = U;
  a.out = H;
  a.ldo = D.f;
  if (tall) return launch_expert<EPI_GLU, ExpertUpPipe2>(D, a, T, s);
  return launch_expert<EPI_GLU>(D, a, T, s);
}

hipError_t launch_expert_down(const Dims& D, const void* H, const int2* tile_info, const int32_t* n_mtiles, int T,
                              const void* W_d, void* Y, hipStream_t s) {
  constexpr int BN = ExpertDownPipe<true>::BN, RB = ExpertDownPipe<true>::RB;
  const int es = esz(D);
  ExpertArgs a{};
  a.A = static_cast<const char*>(H);
  a.lda_bytes = D.f * es;
  a.W = static_cast<const char*>(W_d);
  a.Wu = nullptr;
  a.ldb_bytes = D.f * es;
  a.w_expert_bytes = (size_t)D.l * D.f * es;
  a.N = D.l;
  a.NT = (D.l + BN - 1) / BN;
  a.kt = D.f * es / RB;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.out = Y;
  a.ldo = D.l;
  return launch_expert<EPI_STORE, ExpertDownPipe>(D, a, T, s);
}

// ------------------------------------------------------ backward launchers --
hipError_t launch_dense_nt(const Dims& D, int tag, const void* A, int lda_bytes, int M, int K_bytes,
                           const DenseSegSpec* segs, int nseg, int ldb_bytes, hipStream_t s) {
  constexpr int BM = DensePipe<true>::BM, BN = DensePipe<true>::BN, RB = DensePipe<true>::RB;
  if (nseg < 1 || nseg > 3 || K_bytes <= 0 || K_bytes % RB || lda_bytes % 16 || ldb_bytes % 16)
    return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  DenseArgs a{};
  a.A[0] = static_cast<const char*>(A);
  a.lda_bytes[0] = lda_bytes;
  a.ldb_bytes[0] = ldb_bytes;
  a.kt[0] = K_bytes / RB;
  a.kt[1] = 0;
  a.M = M;
  a.m_tiles = (M + BM - 1) / BM;
  a.nseg = nseg;
  a.total_ntiles = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].kind != EPI_F32 && segs[i].kind != EPI_STORE) return hipErrorInvalidValue;
    DenseSeg& g = a.seg[i];
    g.B[0] = static_cast<const char*>(segs[i].B);
    g.N = segs[i].N;
    g.ntiles = (segs[i].N + BN - 1) / BN;
    g.kind = segs[i].kind;
    g.out = segs[i].out;
    g.ldo = segs[i].ldo;
    g.col_off = nullptr;
    a.total_ntiles += g.ntiles;
  }
  if (tag != 3) return hipErrorInvalidValue;
  return launch_dense_any<3>(D, a, s);
}

hipError_t launch_expert_nt(const Dims& D, const void* A, int lda_bytes, const int32_t* gather, const void* W,
                            size_t w_expert_bytes, int ldb_bytes, int N, int K_bytes, const int2* tile_info,
                            const int32_t* n_mtiles, int T, void* out, int ldo, hipStream_t s) {
  constexpr int BN = ExpertPipe<true>::BN, RB = ExpertPipe<true>::RB;
  if (K_bytes <= 0 || K_bytes % RB || lda_bytes % 16 || ldb_bytes % 16) return hipErrorInvalidValue;
  ExpertArgs a{};
  a.A = static_cast<const char*>(A);
  a.lda_bytes = lda_bytes;
  a.gather = gather;
  a.W = static_cast<const char*>(W);
  a.Wu = nullptr;
  a.ldb_bytes = ldb_bytes;
  a.w_expert_bytes = w_expert_bytes;
  a.N = N;
  a.NT = (N + BN - 1) / BN;
  a.kt = K_bytes / RB;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.out = out;
  a.ldo = ldo;
  return launch_expert<EPI_STORE>(D, a, T, s);
}

// K pieces -> stage boundaries of a pipeline with rb-byte stage rows; false
// if a piece is not whole stages (spans are multiples of 64 values, which
// every stage depth here divides) or is malformed.
static bool dgrad_pieces(const Dims& D, int rb, const KPiece* pc, int npiece, DgradArgs& a, DgradSeg& g) {
  const int kr = rb / esz(D), ce = 16 / esz(D);
  if (npiece < 1 || npiece > 4 || 64 % kr) return false;
  int st = 0;
  for (int j = 0; j < 4; ++j) {
    if (j < npiece) {
      if (pc[j].span <= 0 || pc[j].span % 64 || pc[j].rows < 0 || pc[j].rows > pc[j].span || !pc[j].B ||
          pc[j].ldb % ce || ((uintptr_t)pc[j].B & 15))
        return false;
      a.st[j] = st;
      a.rows[j] = pc[j].rows;
      g.B[j] = static_cast<const char*>(pc[j].B);
      g.ldb[j] = pc[j].ldb;
      st += pc[j].span / kr;
    } else {
      a.st[j] = st;
      a.rows[j] = 0;
      g.B[j] = static_cast<const char*>(pc[0].B);
      g.ldb[j] = pc[0].ldb;
    }
  }
  a.st[4] = st;
  a.npiece = npiece;
  return true;
}

template <bool EXPERT, int TAG>
static hipError_t launch_dgrad_any(const Dims& D, const DgradArgs& a, long long tiles, hipStream_t s) {
  if (tiles == 0) return hipSuccess;
  if (EXPERT) {
    if (D.bf16)
      hipLaunchKernelGGL((k_gemm_dgrad<DgradExpertPipe<true>, true, TAG>),
                         dim3(persistent_grid(tiles, DgradExpertPipe<true>::BPC)), dim3(DgradExpertPipe<true>::THREADS),
                         0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_dgrad<DgradExpertPipe<false>, true, TAG>),
                         dim3(persistent_grid(tiles, DgradExpertPipe<false>::BPC)),
                         dim3(DgradExpertPipe<false>::THREADS), 0, s, a);
  } else {
    if (D.bf16)
      hipLaunchKernelGGL((k_gemm_dgrad<DgradPipe<true>, false, TAG>), dim3(persistent_grid(tiles, DgradPipe<true>::BPC)),
                         dim3(DgradPipe<true>::THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_dgrad<DgradPipe<false>, false, TAG>),
                         dim3(persistent_grid(tiles, DgradPipe<false>::BPC)), dim3(DgradPipe<false>::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dgrad_dense(const Dims& D, int tag, const void* A, int lda_bytes, int M, const DgradSegSpec* segs,
                              int nseg, int npiece, hipStream_t s) {
  constexpr int BM = DgradPipe<true>::BM, BN = DgradPipe<true>::BN;
  if (nseg < 1 || nseg > 2 || !A || lda_bytes % 16 || ((uintptr_t)A & 15)) return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  DgradArgs a{};
  a.A = static_cast<const char*>(A);
  a.lda_bytes = lda_bytes;
  a.M = M;
  a.m_tiles = (M + BM - 1) / BM;
  a.nseg = nseg;
  a.es = esz(D);
  for (int i = 0; i < nseg; ++i) {
    DgradArgs b{};
    DgradSeg& g = a.seg[i];
    if (!dgrad_pieces(D, DgradPipe<true>::RB, segs[i].piece, npiece, b, g)) return hipErrorInvalidValue;
    if (i == 0) {
      std::memcpy(a.st, b.st, sizeof a.st);
      std::memcpy(a.rows, b.rows, sizeof a.rows);
      a.npiece = b.npiece;
    } else if (std::memcmp(a.st, b.st, sizeof a.st) || std::memcmp(a.rows, b.rows, sizeof a.rows)) {
      return hipErrorInvalidValue;  // segments share the K structure
    }
    if (segs[i].N <= 0 || (segs[i].kind != EPI_F32 && segs[i].kind != EPI_STORE) || !segs[i].out)
      return hipErrorInvalidValue;
    g.N = segs[i].N;
    g.ntiles = (segs[i].N + BN - 1) / BN;
    g.kind = segs[i].kind;
    g.out = segs[i].out;
    g.ldo = segs[i].ldo;
    a.total_ntiles += g.ntiles;
  }
  if ((long long)a.st[4] * DgradPipe<true>::RB > lda_bytes) return hipErrorInvalidValue;  // A rows hold all of K
  const long long tiles = (long long)a.m_tiles * a.total_ntiles;
  switch (tag) {
    case 4: return launch_dgrad_any<false, 4>(D, a, tiles, s);
    default: return launch_dgrad_any<false, 5>(D, a, tiles, s);
  }
}

hipError_t launch_dgrad_expert(const Dims& D, int tag, const void* A, int lda_bytes, const KPiece* pieces, int npiece,
                               size_t b_expert_bytes, int N, const int2* tile_info, const int32_t* n_mtiles, int T,
                               void* out, int ldo, hipStream_t s) {
  constexpr int BN = DgradExpertPipe<true>::BN;
  if (!A || lda_bytes % 16 || ((uintptr_t)A & 15) || N <= 0 || !out || b_expert_bytes % 16) return hipErrorInvalidValue;
  DgradArgs a{};
  a.A = static_cast<const char*>(A);
  a.lda_bytes = lda_bytes;
  a.es = esz(D);
  DgradSeg& g = a.seg[0];
  if (!dgrad_pieces(D, DgradExpertPipe<true>::RB, pieces, npiece, a, g)) return hipErrorInvalidValue;
  if ((long long)a.st[4] * DgradExpertPipe<true>::RB > lda_bytes) return hipErrorInvalidValue;
  g.N = N;
  g.ntiles = (N + BN - 1) / BN;
  g.kind = EPI_STORE;
  g.out = out;
  g.ldo = ldo;
  a.nseg = 1;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.b_expert_bytes = b_expert_bytes;
  const long long tiles = (long long)expert_max_mtiles(T, D.k, D.E) * g.ntiles;
  switch (tag) {
    case 8: return launch_dgrad_any<true, 8>(D, a, tiles, s);
    default: return launch_dgrad_any<true, 9>(D, a, tiles, s);
  }
}

hipError_t launch_wgrad_km(const Dims& D, const WgradKmSpec& w, hipStream_t s) {
  constexpr int BM = WgradKmPipe<true>::BM, BN = WgradKmPipe<true>::BN;
  const int es = esz(D), ce = 16 / es;  // elements per 16-byte chunk
  auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (w.M <= 0 || w.N <= 0 || w.nseg < 0 || !w.A || !w.B1 || !w.out || (w.nsplit > 0 && !w.B0) ||
      w.nsplit < 0 || w.nsplit % ce || w.lda % ce || w.ldb0 % ce || w.ldb1 % ce || !al(w.A) || !al(w.B0) ||
      !al(w.B1) || (!w.koff && w.kstep <= 0) || (w.gather && w.ngather <= 0))
    return hipErrorInvalidValue;
  WgradKmArgs a{};
  a.A = static_cast<const char*>(w.A);
  a.B[0] = static_cast<const char*>(w.nsplit > 0 ? w.B0 : w.B1);
  a.B[1] = static_cast<const char*>(w.B1);
  a.lda = w.lda;
  a.ldb[0] = w.nsplit > 0 ? w.ldb0 : w.ldb1;
  a.ldb[1] = w.ldb1;
  a.koff = w.koff;
  a.gather = w.gather;
  a.kstep = w.kstep;
  a.kend = w.kend;
  a.ngather = w.ngather;
  a.nsplit = w.nsplit;
  a.es = es;
  a.M = w.M;
  a.N = w.N;
  a.MT = (w.M + BM - 1) / BM;
  a.NT = (w.N + BN - 1) / BN;
  a.E = w.nseg;
  a.out = w.out;
  const long long tiles = (long long)a.E * a.MT * a.NT;
  if (tiles == 0) return hipSuccess;
  if (D.bf16)
    hipLaunchKernelGGL(k_gemm_wgrad_km<WgradKmPipe<true>>, dim3(persistent_grid(tiles, WgradKmPipe<true>::BPC)),
                       dim3(WgradKmPipe<true>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm_wgrad_km<WgradKmPipe<false>>, dim3(persistent_grid(tiles, WgradKmPipe<false>::BPC)),
                       dim3(WgradKmPipe<false>::THREADS), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- MXFP8 --
hipError_t launch_mx_quant(const void* src, long long rows, int K, long long ld_src, uint8_t* dst, uint8_t* scales,
                           hipStream_t s, bool w4) {
  if (K % 32 || ld_src % 8) return hipErrorInvalidValue;
  const long long n = rows * (K / 32);
  if (n == 0) return hipSuccess;
  if (w4)
    hipLaunchKernelGGL(k_mx_quant<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), rows, K, ld_src, dst, scales);
  else
    hipLaunchKernelGGL(k_mx_quant<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), rows, K, ld_src, dst, scales);
  return hipGetLastError();
}

#ifndef MOE_EXPERT_MX4_CFG
#define MOE_EXPERT_MX4_CFG kExpertBM, 256, 1, 4, 2, 2
#endif
using ExpertMx4Pipe = Mx4Pipe<MOE_EXPERT_MX4_CFG>;
static_assert(ExpertMx4Pipe::BN == ExpertMxPipe::BN, "one weight-row tiling for both block-scaled formats");

template <int KIND>
static hipError_t launch_expert_mx(const Dims& D, const ExpertArgs& a, int T, hipStream_t s, bool w4) {
  const long long tiles = (long long)expert_max_mtiles(T, D.k, D.E) * a.NT;
  if (tiles == 0) return hipSuccess;
  if (w4) {
    using P = ExpertMx4Pipe;
    hipLaunchKernelGGL((k_gemm_expert_mx4<P, KIND>), dim3(persistent_grid(tiles, P::BPC)), dim3(P::THREADS), 0, s,
                       a);
  } else {
    using P = ExpertMxPipe;
    hipLaunchKernelGGL((k_gemm_expert_mx<P, KIND>), dim3(persistent_grid(tiles, P::BPC)), dim3(P::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_expert_up_mx(const Dims& D, const uint8_t* z8, const uint8_t* Xs, const int32_t* perm_src,
                               const int2* tile_info, const int32_t* n_mtiles, int T, const uint8_t* Wg8,
                               const uint8_t* Wgs, const uint8_t* Wu8, const uint8_t* Wus, void* H, uint8_t* H8,
                               uint8_t* Hs, hipStream_t s, bool w4) {
  constexpr int BN = ExpertMxPipe::BN, RB = ExpertMxPipe::RB;
  if (D.l % RB || D.l > 4 * RB) return hipErrorInvalidValue;
  const int wb = w4 ? D.l / 2 : D.l;  // weight row bytes
  ExpertArgs a{};
  a.A = reinterpret_cast<const char*>(z8);
  a.lda_bytes = D.l;
  a.gather = perm_src;
  a.W = reinterpret_cast<const char*>(Wg8);
  a.Wu = reinterpret_cast<const char*>(Wu8);
  a.ldb_bytes = wb;
  a.w_expert_bytes = (size_t)D.f * wb;
  a.N = D.f;
  a.NT = (2 * D.f + BN - 1) / BN;
  a.kt = D.l / RB;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.out = H;
  a.ldo = D.f;
  a.sA = Xs;
  a.sW = Wgs;
  a.sWu = Wus;
  a.s_ld = D.l / 32;
  a.w_rows = D.f;
  a.keep[0] = H8;  // H quantised to MXFP8 in the epilogue
  a.keep[1] = Hs;
  if (!H8 || !Hs) return hipErrorInvalidValue;
  return launch_expert_mx<EPI_GLU_MX>(D, a, T, s, w4);
}

hipError_t launch_expert_down_mx(const Dims& D, const uint8_t* H8, const uint8_t* Hs, const int2* tile_info,
                                 const int32_t* n_mtiles, int T, const uint8_t* Wd8, const uint8_t* Wds, void* Y,
                                 hipStream_t s, bool w4) {
  constexpr int BN = ExpertMxPipe::BN, RB = ExpertMxPipe::RB;
  if (D.f % RB || D.f > 4 * RB) return hipErrorInvalidValue;
  const int wb = w4 ? D.f / 2 : D.f;  // weight row bytes
  ExpertArgs a{};
  a.A = reinterpret_cast<const char*>(H8);
  a.lda_bytes = D.f;
  a.gather = nullptr;
  a.W = reinterpret_cast<const char*>(Wd8);
  a.Wu = nullptr;
  a.ldb_bytes = wb;
  a.w_expert_bytes = (size_t)D.l * wb;
  a.N = D.l;
  a.NT = (D.l + BN - 1) / BN;
  a.kt = D.f / RB;
  a.tile_info = tile_info;
  a.n_mtiles = n_mtiles;
  a.out = Y;
  a.ldo = D.l;
  a.sA = Hs;
  a.sW = Wds;
  a.sWu = nullptr;
  a.s_ld = D.f / 32;
  a.w_rows = D.l;
  return launch_expert_mx<EPI_STORE>(D, a, T, s, w4);
}

}  // namespace moe
