// MFMA GEMMs of the LatentMoE layer on gfx950 (CDNA4).
//
// All products here are y = a W^T with both operands K-contiguous (activation
// rows and PyTorch-layout [out, in] weight rows), fp32 accumulation:
//   * gemm_h:      h [T,d] against [W_r | W_sg,W_su | W_dn] -> fp32 router
//                  logits, the shared GLU hidden G = silu(h W_sg^T)*(h W_su^T)
//                  and the latent z = h W_dn^T in one launch (one pass of h);
//   * expert_up:   per expert, rows z[perm_src] (gathered in the A loader)
//                  against W_g[e], W_u[e] with the GLU in the epilogue -> H;
//   * expert_down: per expert, H rows against W_d[e] -> Y;
//   * gemm_out:    [G | y_lat] against [W_sd | W_up] (one K loop over both
//                  parts) -> out, so the shared and routed paths are summed in
//                  the fp32 accumulators.
// (Width separation and the shared/routed dual path: architecture paragraph
// and Tab 1 of the "Kimi K3 MoE lightweight replica demo" article; the expert
// GLUs as batched matmuls per expert group: capsule 20 of the "Pretraining a
// Mini Kimi K3" review.)
//
// Tiling: 256 threads = 4 wavefronts in a 2x2 grid over a BM x BN block tile;
// K advances 128 bytes per stage (64 bf16 or 32 fp32).  Stages are
// double-buffered in LDS; the next stage's global loads are in flight while
// the current one feeds the MFMAs.  bf16 uses v_mfma_f32_16x16x32_bf16, fp32
// four v_mfma_f32_16x16x4_f32 per 16-byte fragment.  The weight fragment is
// the MFMA's first operand, so each lane's accumulators hold 4 consecutive
// output columns of one row (8- or 16-byte stores).  LDS rows are 128 bytes
// with 16-byte chunks XOR-swizzled by row, so the 16 rows a fragment read
// touches fall in distinct banks.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // K bytes per stage

enum EpiKind { EPI_F32 = 0, EPI_STORE = 1, EPI_GLU = 2 };

MOE_DEV int lds_off(int row, int chunk) {
  const int sw = (row & 7) ^ ((row >> 3) & 1);
  return row * kRowBytes + ((chunk ^ sw) << 4);
}

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
// add a wait for all outstanding loads before every LDS read; the loop below
// waits for its own loads explicitly.
MOE_DEV void lds_dma16(const char* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

// Stage filling: a stage is BM + BN rows of 128 bytes (A rows, then B rows),
// written by 1 KB DMA slots; thread (wave w, lane) fills slots i*4 + w, i < L.
// The tile row and the logical 16-byte K chunk that a lane's piece of slot i
// holds (the LDS chunk position is lane%8, XOR-swizzled by row):
MOE_DEV int slot_row(int i, int wave, int lane) { return (i * 4 + wave) * 8 + (lane >> 3); }
MOE_DEV int slot_chunk(int row, int lane) { return (lane & 7) ^ ((row & 7) ^ ((row >> 3) & 1)); }

// Global source of each of this thread's slot pieces at k = 0, per K part;
// the source advances 128 bytes per stage.  PARTS K parts are consumed one
// after the other (kt[p] stages each).
template <int L, int PARTS>
struct Src {
  const char* p[PARTS][L];
  int kt[PARTS];
};

template <int BM, int BN, bool BF16>
struct Core {
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int MI = WTM / 16, NI = WTN / 16;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int L = STAGE / 1024 / 4;  // DMA slots per thread per stage
  static_assert(STAGE % 4096 == 0, "stage must split into 1 KB slots over 4 wavefronts");

  // Accumulate all stages into acc.  Two LDS buffers: the loads of stage s+1
  // are issued right after the barrier that ends stage s-1's reads, and run
  // while stage s feeds the MFMAs.
  template <int PARTS>
  MOE_DEV static void run(const Src<L, PARTS>& S, f32x4_t (&acc)[MI][NI], char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int KT = S.kt[0];
    if constexpr (PARTS > 1) KT += S.kt[1];
    if (KT <= 0) return;
    const uint32_t lds0 = lds_addr(smem) + wave * 1024;
    auto issue = [&](int s, int buf) {
      bool second = false;
      int ks = s;
      if constexpr (PARTS > 1) {
        second = s >= S.kt[0];
        ks = second ? s - S.kt[0] : s;
      }
      const uint32_t base = lds0 + buf * STAGE;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const char* g = S.p[0][i];
        if constexpr (PARTS > 1) g = second ? S.p[1][i] : g;
        lds_dma16(g + ks * kRowBytes, __builtin_amdgcn_readfirstlane(base + i * 4096));
      }
    };
    issue(0, 0);
    for (int s = 0; s < KT; ++s) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (s + 1 < KT) issue(s + 1, (s + 1) & 1);
      const char* cur = smem + (s & 1) * STAGE;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ch = kk * 4 + (lane >> 4);
        uint4 af[MI], wf[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          af[mi] = *reinterpret_cast<const uint4*>(cur + lds_off(wm * WTM + mi * 16 + (lane & 15), ch));
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          wf[ni] = *reinterpret_cast<const uint4*>(cur + A_BYTES + lds_off(wn * WTN + ni * 16 + (lane & 15), ch));
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) mfma_chunk<BF16>(acc[mi][ni], wf[ni], af[mi]);
      }
    }
  }

  MOE_DEV static void zero(f32x4_t (&acc)[MI][NI]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
  //   EPI_F32:   fp32 store (+ per-column offset), columns < N only.
  //   EPI_STORE: store in the activation dtype (N a multiple of 4).
  //   EPI_GLU:   tile columns alternate 16 gate / 16 up; output column
  //              n0/2 + 16*(c/32) + c%16 gets silu(gate) * up.
  template <int KIND>
  MOE_DEV static void epilogue(const f32x4_t (&acc)[MI][NI], int rows_valid, int n0, int N, void* out, int ldo,
                               size_t row_base, const float* col_off) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
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
          for (int r = 0; r < 4; ++r) o[r] = g[r] / (1.0f + __expf(-g[r])) * u[r];
          store4(out, orow + c, o[0], o[1], o[2], o[3]);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int c = n0 + wn * WTN + ni * 16 + 4 * (lane >> 4);
          const f32x4_t v = acc[mi][ni];
          if constexpr (KIND == EPI_F32) {
            float* o = static_cast<float*>(out) + orow;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (c + r < N) o[c + r] = v[r] + (col_off ? col_off[c + r] : 0.f);
          } else {
            if (c < N) store4(out, orow + c, v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
};

// ------------------------------------------------------------ dense GEMMs --
struct DenseSeg {
  const char* B[2];   // weight rows of K part 0 / 1 (gate rows for a GLU)
  const char* Bu[2];  // up rows for a GLU
  int N;              // output columns
  int ntiles;
  int kind;
  void* out;
  int ldo;
  const float* col_off;
};

struct DenseArgs {
  const char* A[2];
  int lda_bytes[2];
  int ldb_bytes[2];
  int kt[2];  // stages per K part
  int M, m_tiles;
  int nseg, total_ntiles;
  DenseSeg seg[3];
};

constexpr int kGroupM = 8;

template <int BM, int BN, bool BF16>
__global__ __launch_bounds__(kThreads) void k_gemm_dense(const DenseArgs args) {
  using C = Core<BM, BN, BF16>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int nblocks = args.m_tiles * args.total_ntiles;
  const int L = xcd_remap(blockIdx.x, nblocks);
  // groups of kGroupM m-tiles, m fastest inside a group
  const int per_group = kGroupM * args.total_ntiles;
  const int group = L / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(args.m_tiles - first_m, kGroupM);
  const int in_group = L - group * per_group;
  const int mt = first_m + in_group % gm;
  int nt = in_group / gm;
  // segment of this n-tile (selects, not a dynamic index into the kernel
  // argument, so the descriptor stays in scalar registers)
  DenseSeg S = args.seg[0];
  if (args.nseg > 1 && nt >= args.seg[0].ntiles) {
    nt -= args.seg[0].ntiles;
    S = args.seg[1];
    if (args.nseg > 2 && nt >= args.seg[1].ntiles) {
      nt -= args.seg[1].ntiles;
      S = args.seg[2];
    }
  }
  const int m0 = mt * BM;
  const int rows_valid = min(BM, args.M - m0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Src<C::L, 2> src;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    src.kt[part] = args.kt[part];
#pragma unroll
    for (int i = 0; i < C::L; ++i) {
      const int row = slot_row(i, wave, lane);
      const int chunk = slot_chunk(row, lane);
      const char* p;
      if (row < BM) {  // A row (rows past the end read row m0: their results are not stored)
        const int r = row < rows_valid ? row : 0;
        p = args.A[part] + (size_t)(m0 + r) * args.lda_bytes[part];
      } else {         // weight row of output column c (columns past N read row 0)
        const int c = row - BM;
        int wrow;
        const char* base;
        if (S.kind == EPI_GLU) {
          wrow = nt * (BN / 2) + (c >> 5) * 16 + (c & 15);
          base = ((c & 31) >= 16) ? S.Bu[part] : S.B[part];
        } else {
          wrow = nt * BN + c;
          base = S.B[part];
        }
        if (wrow >= S.N) wrow = 0;
        p = base + (size_t)wrow * args.ldb_bytes[part];
      }
      src.p[part][i] = args.kt[part] > 0 ? p + chunk * 16 : nullptr;
    }
  }
  f32x4_t acc[C::MI][C::NI];
  C::zero(acc);
  C::template run<2>(src, acc, smem);
  if (S.kind == EPI_F32)
    C::template epilogue<EPI_F32>(acc, rows_valid, nt * BN, S.N, S.out, S.ldo, (size_t)m0, S.col_off);
  else if (S.kind == EPI_GLU)
    C::template epilogue<EPI_GLU>(acc, rows_valid, nt * BN, S.N, S.out, S.ldo, (size_t)m0, nullptr);
  else
    C::template epilogue<EPI_STORE>(acc, rows_valid, nt * BN, S.N, S.out, S.ldo, (size_t)m0, nullptr);
}

// ---------------------------------------------------------- expert GEMMs --
// Tile decode: logical tile L -> global m-tile L / NT (owned by the expert e
// with tile_offsets[e] <= L/NT < tile_offsets[e+1], found by binary search)
// and n-tile L % NT.  The grid is an upper bound; blocks past the device-side
// tile count exit at once.
MOE_DEV int find_expert(const int32_t* __restrict__ tile_offsets, int E, int gmt) {
  int lo = 0, hi = E - 1;  // largest e with tile_offsets[e] <= gmt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_offsets[mid] <= gmt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct ExpertArgs {
  const char* A;            // z (up) or H (down)
  const int32_t* perm_src;  // gather rows through it (up) or nullptr (down)
  int src_rows;             // rows of A
  int lda_bytes;
  const char* W;   // W_g (up) or W_d (down), [E, N, K]
  const char* Wu;  // W_u (up) or nullptr
  int ldb_bytes;
  size_t w_expert_bytes;
  int N;  // output columns
  int NT;
  int kt;
  const int32_t* offsets;
  const int32_t* tile_offsets;
  int E;
  void* out;
  int ldo;
};

template <int BN, bool BF16, int KIND>
__global__ __launch_bounds__(kThreads) void k_gemm_expert(const ExpertArgs args) {
  constexpr int BM = kExpertBM;
  using C = Core<BM, BN, BF16>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int total = args.tile_offsets[args.E] * args.NT;
  if ((int)blockIdx.x >= total) return;
  const int L = xcd_remap(blockIdx.x, total);
  const int gmt = L / args.NT, nt = L - gmt * args.NT;
  const int e = find_expert(args.tile_offsets, args.E, gmt);
  const int mt = gmt - args.tile_offsets[e];
  const int row0 = args.offsets[e] + mt * BM;
  const int rows_valid = min(BM, args.offsets[e + 1] - row0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* Wg = args.W + (size_t)e * args.w_expert_bytes;
  const char* Wu = args.Wu ? args.Wu + (size_t)e * args.w_expert_bytes : nullptr;
  Src<C::L, 1> src;
  src.kt[0] = args.kt;
#pragma unroll
  for (int i = 0; i < C::L; ++i) {
    const int row = slot_row(i, wave, lane);
    const int chunk = slot_chunk(row, lane);
    const char* p;
    if (row < BM) {  // rows past the expert's end read its first row (results not stored)
      const int r = row0 + (row < rows_valid ? row : 0);
      int srow = args.perm_src ? args.perm_src[r] : r;
      srow = (unsigned)srow < (unsigned)args.src_rows ? srow : 0;  // never taken for a consistent permutation
      p = args.A + (size_t)srow * args.lda_bytes;
    } else {
      const int c = row - BM;
      int wrow;
      const char* base;
      if (KIND == EPI_GLU) {
        wrow = nt * (BN / 2) + (c >> 5) * 16 + (c & 15);
        base = ((c & 31) >= 16) ? Wu : Wg;
      } else {
        wrow = nt * BN + c;
        base = Wg;
      }
      if (wrow >= args.N) wrow = 0;
      p = base + (size_t)wrow * args.ldb_bytes;
    }
    src.p[0][i] = p + chunk * 16;
  }
  f32x4_t acc[C::MI][C::NI];
  C::zero(acc);
  C::template run<1>(src, acc, smem);
  C::template epilogue<KIND>(acc, rows_valid, nt * BN, args.N, args.out, args.ldo, (size_t)row0, nullptr);
}

constexpr int kDenseBM = 128, kDenseBN = 128;
constexpr int kExpertBN = 128;

}  // namespace

static int esz(const Dims& D) { return D.bf16 ? 2 : 4; }

template <bool BF16>
static hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  const int nblocks = a.m_tiles * a.total_ntiles;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_dense<kDenseBM, kDenseBN, BF16>), dim3(nblocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_h(const Dims& D, const void* h, int T, const void* W_r, const float* logit_offset,
                         const void* W_sg, const void* W_su, const void* W_dn, float* logits, void* G, void* z,
                         hipStream_t s) {
  const int es = esz(D);
  DenseArgs a{};
  a.A[0] = static_cast<const char*>(h);
  a.lda_bytes[0] = D.d * es;
  a.ldb_bytes[0] = D.d * es;
  a.kt[0] = D.d * es / kRowBytes;
  a.kt[1] = 0;
  a.M = T;
  a.m_tiles = (T + kDenseBM - 1) / kDenseBM;
  int ns = 0;
  if (logits) {  // router logits, fp32
    DenseSeg& g = a.seg[ns++];
    g.B[0] = static_cast<const char*>(W_r);
    g.N = D.E;
    g.ntiles = (D.E + kDenseBN - 1) / kDenseBN;
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
    g.ntiles = (2 * D.f_s + kDenseBN - 1) / kDenseBN;
    g.kind = EPI_GLU;
    g.out = G;
    g.ldo = D.f_s;
  }
  if (z) {  // latent z
    DenseSeg& g = a.seg[ns++];
    g.B[0] = static_cast<const char*>(W_dn);
    g.N = D.l;
    g.ntiles = (D.l + kDenseBN - 1) / kDenseBN;
    g.kind = EPI_STORE;
    g.out = z;
    g.ldo = D.l;
  }
  if (ns == 0) return hipSuccess;
  a.nseg = ns;
  a.total_ntiles = 0;
  for (int i = 0; i < ns; ++i) a.total_ntiles += a.seg[i].ntiles;
  return D.bf16 ? launch_dense<true>(a, s) : launch_dense<false>(a, s);
}

hipError_t launch_gemm_out(const Dims& D, const void* G, const void* y_lat, int T, const void* W_sd,
                           const void* W_up, void* out, hipStream_t s) {
  const int es = esz(D);
  DenseArgs a{};
  int p = 0;
  if (D.f_s > 0) {
    a.A[p] = static_cast<const char*>(G);
    a.lda_bytes[p] = D.f_s * es;
    a.ldb_bytes[p] = D.f_s * es;
    a.kt[p] = D.f_s * es / kRowBytes;
    a.seg[0].B[p] = static_cast<const char*>(W_sd);
    ++p;
  }
  a.A[p] = static_cast<const char*>(y_lat);
  a.lda_bytes[p] = D.l * es;
  a.ldb_bytes[p] = D.l * es;
  a.kt[p] = D.l * es / kRowBytes;
  a.seg[0].B[p] = static_cast<const char*>(W_up);
  a.M = T;
  a.m_tiles = (T + kDenseBM - 1) / kDenseBM;
  a.seg[0].N = D.d;
  a.seg[0].ntiles = (D.d + kDenseBN - 1) / kDenseBN;
  a.seg[0].kind = EPI_STORE;
  a.seg[0].out = out;
  a.seg[0].ldo = D.d;
  a.nseg = 1;
  a.total_ntiles = a.seg[0].ntiles;
  return D.bf16 ? launch_dense<true>(a, s) : launch_dense<false>(a, s);
}

static int expert_grid(const Dims& D, int T, int NT) {
  // sum_e ceil(n_e / BM) <= T*k/BM + E (at most one partial tile per expert)
  const long long tiles = ((long long)T * D.k + kExpertBM - 1) / kExpertBM + D.E;
  return (int)(tiles * NT);
}

hipError_t launch_expert_up(const Dims& D, const void* z, const int32_t* perm_src, const int32_t* offsets,
                            const int32_t* tile_offsets, int T, const void* W_g, const void* W_u, void* H,
                            hipStream_t s) {
  const int es = esz(D);
  ExpertArgs a{};
  a.A = static_cast<const char*>(z);
  a.perm_src = perm_src;
  a.src_rows = T;
  a.lda_bytes = D.l * es;
  a.W = static_cast<const char*>(W_g);
  a.Wu = static_cast<const char*>(W_u);
  a.ldb_bytes = D.l * es;
  a.w_expert_bytes = (size_t)D.f * D.l * es;
  a.N = D.f;
  a.NT = (2 * D.f + kExpertBN - 1) / kExpertBN;
  a.kt = D.l * es / kRowBytes;
  a.offsets = offsets;
  a.tile_offsets = tile_offsets;
  a.E = D.E;
  a.out = H;
  a.ldo = D.f;
  const int grid = expert_grid(D, T, a.NT);
  if (grid == 0) return hipSuccess;
  if (D.bf16)
    hipLaunchKernelGGL((k_gemm_expert<kExpertBN, true, EPI_GLU>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_expert<kExpertBN, false, EPI_GLU>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expert_down(const Dims& D, const void* H, const int32_t* offsets, const int32_t* tile_offsets,
                              int T, const void* W_d, void* Y, hipStream_t s) {
  const int es = esz(D);
  ExpertArgs a{};
  a.A = static_cast<const char*>(H);
  a.perm_src = nullptr;
  a.src_rows = T * D.k;
  a.lda_bytes = D.f * es;
  a.W = static_cast<const char*>(W_d);
  a.Wu = nullptr;
  a.ldb_bytes = D.f * es;
  a.w_expert_bytes = (size_t)D.l * D.f * es;
  a.N = D.l;
  a.NT = (D.l + kExpertBN - 1) / kExpertBN;
  a.kt = D.f * es / kRowBytes;
  a.offsets = offsets;
  a.tile_offsets = tile_offsets;
  a.E = D.E;
  a.out = Y;
  a.ldo = D.l;
  const int grid = expert_grid(D, T, a.NT);
  if (grid == 0) return hipSuccess;
  if (D.bf16)
    hipLaunchKernelGGL((k_gemm_expert<kExpertBN, true, EPI_STORE>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_expert<kExpertBN, false, EPI_STORE>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
