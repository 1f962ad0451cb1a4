// Dense bf16 contractions on CDNA4 MFMA (v_mfma_f32_16x16x32_bf16):
//  G1  up-projection  z = x w_up_t^T + b, h = ReLU(z) rounded to bf16, with the
//      TwELL pack of every (row, tile) of h fused into the epilogue;
//  G4  dense fallback y[dense_rows[m]] = dense_values[m] w_down.
//
// The TwELL format and its hybrid dense fallback follow "Sparser, Faster,
// Lighter Transformer Language Models (Sakana AI + NVIDIA)", Figure 1
// description; the fusion of the format into the MLP kernels follows
// "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse Transformers Run Like
// They Were Built for Hopper", section "TwELL: The Packing Format That Fits
// the Machine" (every extra pass over memory costs the gains).
//
// Block tile BM x BN x 64 (K), 256 threads = 4 waves arranged WAVES_M x
// WAVES_N, each wave owning a (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of
// 16x16 MFMA blocks.  Operands are staged global -> registers -> LDS with a
// one-tile register prefetch; LDS rows are K-contiguous with a 16-byte pad so
// the 16-byte fragment reads of 16 consecutive rows hit distinct banks.
// A B operand stored [K][N] (w_down) is transposed 8x8 in registers while
// staging, so both operands are read from LDS the same way.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "spmm_split.h"

namespace twell {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS pitch (elements) of a K-contiguous operand row

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int A_VECS = BM * BK / 8 / kThreads;  // 16-byte vectors per thread
  static constexpr int B_VECS = BN * BK / 8 / kThreads;
  static constexpr int B_BLOCKS = (BN / 8) * (BK / 8);    // 8x8 blocks of a [K][N] operand
  static constexpr int B_BLK_PER_THREAD = (B_BLOCKS + kThreads - 1) / kThreads;
  static constexpr int LDS_ELEMS = (BM + BN) * LDK;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per block");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile of 16x16 blocks");
  static_assert(A_VECS * kThreads * 8 == BM * BK, "A tile splits evenly");
  static_assert(B_VECS * kThreads * 8 == BN * BK, "B tile splits evenly");
};

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Operand rows [r0, r0 + ROWS) x K-columns [k0, k0 + 64) of a K-contiguous
// matrix (row pitch ld), rows >= nrows or columns >= K read as zero.
template <int ROWS, int VECS>
__device__ __forceinline__ void load_k_major(const uint16_t* __restrict__ src, int64_t ld,
                                             int nrows, int r0, int K, int k0, uint4 (&reg)[VECS]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < VECS; ++i) {
    const int v = tid + i * kThreads;
    const int row = v / (BK / 8);
    const int kv = v % (BK / 8);
    const int gr = r0 + row;
    const int gk = k0 + kv * 8;
    if (gr < nrows && gk < K)
      reg[i] = load16(src + static_cast<int64_t>(gr) * ld + gk);
    else
      reg[i] = make_uint4(0, 0, 0, 0);
  }
}

template <int VECS>
__device__ __forceinline__ void store_k_major(uint16_t* __restrict__ lds, const uint4 (&reg)[VECS]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < VECS; ++i) {
    const int v = tid + i * kThreads;
    const int row = v / (BK / 8);
    const int kv = v % (BK / 8);
    *reinterpret_cast<uint4*>(lds + row * LDK + kv * 8) = reg[i];
  }
}

// An operand stored [K][N] (N contiguous, row pitch ld): each thread loads
// 8x8 blocks (8 K-rows of 8 consecutive N), for columns [n0, n0 + BN).
template <int BN, int NBLK>
__device__ __forceinline__ void load_n_major(const uint16_t* __restrict__ src, int64_t ld, int N,
                                             int n0, int K, int k0, uint4 (&reg)[NBLK][8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int blk = tid + b * kThreads;
    const int nv = blk % (BN / 8);
    const int kb = blk / (BN / 8);
    const int gn = n0 + nv * 8;
    const bool live = blk < (BN / 8) * (BK / 8) && gn < N;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int gk = k0 + kb * 8 + r;
      if (live && gk < K)
        reg[b][r] = load16(src + static_cast<int64_t>(gk) * ld + gn);
      else
        reg[b][r] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t pick(const uint4& q, int d) {
  return d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
}

// Transpose the 8x8 bf16 blocks and store them K-contiguous: LDS row n holds
// k = kb*8 .. kb*8+7 of column n.
template <int BN, int NBLK>
__device__ __forceinline__ void store_n_major(uint16_t* __restrict__ lds, const uint4 (&reg)[NBLK][8]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int blk = tid + b * kThreads;
    if (blk >= (BN / 8) * (BK / 8)) continue;
    const int nv = blk % (BN / 8);
    const int kb = blk / (BN / 8);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      uint32_t e[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = pick(reg[b][2 * p], n / 2);
        const uint32_t hi = pick(reg[b][2 * p + 1], n / 2);
        e[p] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<uint4*>(lds + (nv * 8 + n) * LDK + kb * 8) = make_uint4(e[0], e[1], e[2], e[3]);
    }
  }
}

// C[BM x BN] += A[m0.., :] * B^T, accumulated in MFMA fragments.
//   A: [M][K] K-contiguous, pitch lda.
//   B: B_NK ? [N][K] K-contiguous (pitch ldb) : [K][N] N-contiguous (pitch ldb).
template <int BM, int BN, int WAVES_M, int WAVES_N, bool B_NK>
__device__ __forceinline__ void mfma_mainloop(
    const uint16_t* __restrict__ A, int64_t lda, int M, int m0, const uint16_t* __restrict__ B,
    int64_t ldb, int N, int n0, int K, uint16_t* __restrict__ sA, uint16_t* __restrict__ sB,
    f32x4_t (&acc)[Tile<BM, BN, WAVES_M, WAVES_N>::FM][Tile<BM, BN, WAVES_M, WAVES_N>::FN]) {
  typedef Tile<BM, BN, WAVES_M, WAVES_N> TL;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[TL::A_VECS];
  uint4 rbk[B_NK ? TL::B_VECS : 1];
  uint4 rbn[B_NK ? 1 : TL::B_BLK_PER_THREAD][8];

  auto load = [&](int k0) {
    load_k_major<BM, TL::A_VECS>(A, lda, M, m0, K, k0, ra);
    if constexpr (B_NK)
      load_k_major<BN, TL::B_VECS>(B, ldb, N, n0, K, k0, rbk);
    else
      load_n_major<BN, TL::B_BLK_PER_THREAD>(B, ldb, N, n0, K, k0, rbn);
  };
  auto store = [&]() {
    store_k_major<TL::A_VECS>(sA, ra);
    if constexpr (B_NK)
      store_k_major<TL::B_VECS>(sB, rbk);
    else
      store_n_major<BN, TL::B_BLK_PER_THREAD>(sB, rbn);
  };

  const int ktiles = (K + BK - 1) / BK;
  load(0);
  store();
  __syncthreads();
  const int arow = wm * TL::WTM + (lane & 15);
  const int brow = wn * TL::WTN + (lane & 15);
  const int kofs = (lane >> 4) * 8;
  for (int kt = 0; kt < ktiles; ++kt) {
    if (kt + 1 < ktiles) load((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t a[TL::FM], b[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(sA + (arow + i * 16) * LDK + ks * 32 + kofs);
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(sB + (brow + j * 16) * LDK + ks * 32 + kofs);
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < ktiles) {
      store();
      __syncthreads();
    }
  }
}

// ============================================================ fast path
// For K a multiple of 64.  K-major operand tiles live in LDS as rows of 64
// K-elements (128 B) without padding; the 16-byte chunk kc of row r sits at
// chunk position kc ^ swz(r) for fragments of 32 rows x 2 chunks (32x32x16
// MFMA) and kc ^ swz16(r) for fragments of 16 rows x 4 chunks (16x16x32), so
// that a wave's fragment load has no LDS bank conflicts.  A K-major operand is
// copied global -> LDS by global_load_lds_dwordx4 (no VGPR staging): one
// instruction of a wave fills one 1 KB block = 8 rows, and lane l fetches the
// global chunk that belongs at LDS position l.  A [K][N] operand (w_down) is
// copied as stored, with 32-byte chunks swizzled by row, and read with LDS
// transpose loads.  Two LDS stages, one barrier per 64-wide K step.
namespace fast {

constexpr int BKF = 64;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
// element offset of (row r, 16-byte chunk kc) inside a swizzled operand tile
__device__ __forceinline__ int tofs(int r, int kc) { return r * BKF + ((kc ^ swz(r)) << 3); }
// Swizzle for operands read as 16-row fragments (16x16x32 MFMA: a wave's read
// covers 16 rows x 4 chunks): row bits 1, 2, 3 go to chunk bits 0, 2, 1.
__device__ __forceinline__ int swz16(int r) { return ((r >> 1) & 1) | (r & 4) | ((r >> 2) & 2); }
__device__ __forceinline__ int tofs16(int r, int kc) { return r * BKF + ((kc ^ swz16(r)) << 3); }

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * kWave;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_ISSUE = BM / (8 * NW);  // DMA instructions per thread per stage
  static constexpr int B_ISSUE = BN / (8 * NW);
  static constexpr int STAGE = (BM + BN) * BKF;                // elements per LDS stage
  static_assert(A_ISSUE * 8 * NW == BM && B_ISSUE * 8 * NW == BN, "whole 1 KB blocks per wave");
  static_assert(FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "16x16 blocks");
};

// Global source of the chunk each lane fetches for DMA instruction i of a
// K-major operand (rows r0.., clamped to nrows-1: rows past the end feed only
// outputs that are never stored).
template <int ISSUE, int NW, bool SW16 = false>
__device__ __forceinline__ void dma_sources(const uint16_t* __restrict__ base, int64_t ld, int nrows,
                                            int r0, const uint16_t* (&src)[ISSUE]) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ISSUE; ++i) {
    const int blk = wave + NW * i;
    const int r = blk * 8 + lane / 8;
    const int kc = (lane & 7) ^ (SW16 ? swz16(r) : swz(r));
    const int gr = min(r0 + r, nrows - 1);
    src[i] = base + static_cast<int64_t>(gr) * ld + kc * 8;
  }
}

template <int ISSUE, int NW>
__device__ __forceinline__ void dma_issue(const uint16_t* const* src, int k0, uint16_t* tile) {
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ISSUE; ++i)
    __builtin_amdgcn_global_load_lds(src[i] + k0, tile + (wave + NW * i) * 512, 16, 0, 0);
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// One LDS stage of C += A B^T on v_mfma_f32_32x32x16_bf16: lane l of a
// fragment holds row (l & 31) and the 8 k's of 16-byte chunk kc = 2 ks + l/32.
template <class CF>
__device__ __forceinline__ void compute_stage32(const uint16_t* __restrict__ sA,
                                                const uint16_t* __restrict__ sB,
                                                f32x16_t (&acc)[CF::WTM / 32][CF::WTN / 32]) {
  constexpr int FM = CF::WTM / 32, FN = CF::WTN / 32;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
#pragma unroll
  for (int ks = 0; ks < BKF / 16; ++ks) {
    const int kc = ks * 2 + (lane >> 5);
    bf16x8_t a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(sA + tofs(wm * CF::WTM + i * 32 + (lane & 31), kc));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t*>(sB + tofs(wn * CF::WTN + j * 32 + (lane & 31), kc));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// C[BM x BN] = A[m0.., :] B[n0.., :]^T, A [M][K] and B [N][K] both K-major,
// K % 64 == 0, both operands copied by DMA.  `lds` holds two stages.
template <class CF>
__device__ __forceinline__ void mainloop32(const uint16_t* __restrict__ A, int64_t lda, int M,
                                           int m0, const uint16_t* __restrict__ B, int64_t ldb,
                                           int N, int n0, int K, uint16_t* lds,
                                           f32x16_t (&acc)[CF::WTM / 32][CF::WTN / 32]) {
#pragma unroll
  for (int i = 0; i < CF::WTM / 32; ++i)
#pragma unroll
    for (int j = 0; j < CF::WTN / 32; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const uint16_t* asrc[CF::A_ISSUE];
  const uint16_t* bsrc[CF::B_ISSUE];
  dma_sources<CF::A_ISSUE, CF::NW>(A, lda, M, m0, asrc);
  dma_sources<CF::B_ISSUE, CF::NW>(B, ldb, N, n0, bsrc);
  const int KT = K / BKF;
  dma_issue<CF::A_ISSUE, CF::NW>(asrc, 0, lds);
  dma_issue<CF::B_ISSUE, CF::NW>(bsrc, 0, lds + CF::BM * BKF);
  for (int kt = 0; kt < KT; ++kt) {
    uint16_t* cur = lds + (kt & 1) * CF::STAGE;
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this thread's copies of tile kt landed
    __syncthreads();  // tile kt visible to all; everyone is done with tile kt-1's stage
    if (kt + 1 < KT) {
      uint16_t* nxt = lds + ((kt + 1) & 1) * CF::STAGE;
      dma_issue<CF::A_ISSUE, CF::NW>(asrc, (kt + 1) * BKF, nxt);
      dma_issue<CF::B_ISSUE, CF::NW>(bsrc, (kt + 1) * BKF, nxt + CF::BM * BKF);
    }
    compute_stage32<CF>(cur, cur + CF::BM * BKF, acc);
  }
  __syncthreads();  // operand stages are free for the epilogue
}

// ---- software-pipelined form of mainloop32 for waves of 64 x 128 (2 x 4
// blocks of 32x32).  Each 16-wide K step is one asm block: the 8 MFMAs of the
// fragments in hand with the 6 ds_reads of the next step's fragments between
// them, and a wait for those reads at its end (so no read is in flight when
// the block ends).  The MFMAs of a stage's last step run after the next
// stage's barrier, beside the reads of its first step.  Same products in the
// same K order as mainloop32, so the same bits.
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

struct Frags24 {
  i32x4_t a[2], b[4];
};

__device__ __forceinline__ void pipe_step(f32x16_t (&c)[2][4], const Frags24& cur, Frags24& nxt,
                                          const uint32_t (&ad)[6]) {
  asm volatile(
      "ds_read_b128 %[na0], %[p0]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"
      "ds_read_b128 %[na1], %[p1]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"
      "ds_read_b128 %[nb0], %[p2]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c02], %[a0], %[b2], %[c02]\n\t"
      "ds_read_b128 %[nb1], %[p3]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c03], %[a0], %[b3], %[c03]\n\t"
      "ds_read_b128 %[nb2], %[p4]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"
      "ds_read_b128 %[nb3], %[p5]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c12], %[a1], %[b2], %[c12]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c13], %[a1], %[b3], %[c13]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [c00] "+v"(c[0][0]), [c01] "+v"(c[0][1]), [c02] "+v"(c[0][2]), [c03] "+v"(c[0][3]),
        [c10] "+v"(c[1][0]), [c11] "+v"(c[1][1]), [c12] "+v"(c[1][2]), [c13] "+v"(c[1][3]),
        [na0] "=&v"(nxt.a[0]), [na1] "=&v"(nxt.a[1]), [nb0] "=&v"(nxt.b[0]),
        [nb1] "=&v"(nxt.b[1]), [nb2] "=&v"(nxt.b[2]), [nb3] "=&v"(nxt.b[3])
      : [a0] "v"(cur.a[0]), [a1] "v"(cur.a[1]), [b0] "v"(cur.b[0]), [b1] "v"(cur.b[1]),
        [b2] "v"(cur.b[2]), [b3] "v"(cur.b[3]), [p0] "v"(ad[0]), [p1] "v"(ad[1]), [p2] "v"(ad[2]),
        [p3] "v"(ad[3]), [p4] "v"(ad[4]), [p5] "v"(ad[5]));
}

__device__ __forceinline__ void pipe_last(f32x16_t (&c)[2][4], const Frags24& cur) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %[c00], %[a0], %[b0], %[c00]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c01], %[a0], %[b1], %[c01]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c02], %[a0], %[b2], %[c02]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c03], %[a0], %[b3], %[c03]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c10], %[a1], %[b0], %[c10]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c11], %[a1], %[b1], %[c11]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c12], %[a1], %[b2], %[c12]\n\t"
      "v_mfma_f32_32x32x16_bf16 %[c13], %[a1], %[b3], %[c13]\n\t"
      : [c00] "+v"(c[0][0]), [c01] "+v"(c[0][1]), [c02] "+v"(c[0][2]), [c03] "+v"(c[0][3]),
        [c10] "+v"(c[1][0]), [c11] "+v"(c[1][1]), [c12] "+v"(c[1][2]), [c13] "+v"(c[1][3])
      : [a0] "v"(cur.a[0]), [a1] "v"(cur.a[1]), [b0] "v"(cur.b[0]), [b1] "v"(cur.b[1]),
        [b2] "v"(cur.b[2]), [b3] "v"(cur.b[3]));
}

__device__ __forceinline__ void pipe_load(Frags24& nxt, const uint32_t (&ad)[6]) {
  asm volatile(
      "ds_read_b128 %[na0], %[p0]\n\t"
      "ds_read_b128 %[na1], %[p1]\n\t"
      "ds_read_b128 %[nb0], %[p2]\n\t"
      "ds_read_b128 %[nb1], %[p3]\n\t"
      "ds_read_b128 %[nb2], %[p4]\n\t"
      "ds_read_b128 %[nb3], %[p5]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [na0] "=&v"(nxt.a[0]), [na1] "=&v"(nxt.a[1]), [nb0] "=&v"(nxt.b[0]),
        [nb1] "=&v"(nxt.b[1]), [nb2] "=&v"(nxt.b[2]), [nb3] "=&v"(nxt.b[3])
      : [p0] "v"(ad[0]), [p1] "v"(ad[1]), [p2] "v"(ad[2]), [p3] "v"(ad[3]), [p4] "v"(ad[4]),
        [p5] "v"(ad[5]));
}

// The accumulators start at `init` (the bias of each column) instead of 0.
template <class CF>
__device__ __forceinline__ void mainloop32_pipe(const uint16_t* __restrict__ A, int64_t lda, int M,
                                                int m0, const uint16_t* __restrict__ B,
                                                int64_t ldb, int N, int n0, int K, uint16_t* lds,
                                                const float (&init)[4], f32x16_t (&acc)[2][4]) {
  static_assert(CF::WTM == 64 && CF::WTN == 128, "2 x 4 blocks of 32x32 per wave");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = init[j];
  // VALU writes of the accumulators, then MFMAs that read them (in asm); the
  // accumulators are operands so the writes cannot move past the wait
  asm volatile("s_nop 15\n\ts_nop 15"
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]),
                 "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3]));
  const uint16_t* asrc[CF::A_ISSUE];
  const uint16_t* bsrc[CF::B_ISSUE];
  dma_sources<CF::A_ISSUE, CF::NW>(A, lda, M, m0, asrc);
  dma_sources<CF::B_ISSUE, CF::NW>(B, ldb, N, n0, bsrc);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)lds));
  // LDS byte addresses of the fragments of each 16-wide K step in stage 0
  uint32_t addr[4][6];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      addr[ks][i] = lbase + 2u * tofs(wm * CF::WTM + i * 32 + (lane & 31), kc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      addr[ks][2 + j] = lbase + 2u * (CF::BM * BKF + tofs(wn * CF::WTN + j * 32 + (lane & 31), kc));
  }
  const int KT = K / BKF;
  Frags24 f0, f1;
  dma_issue<CF::A_ISSUE, CF::NW>(asrc, 0, lds);
  dma_issue<CF::B_ISSUE, CF::NW>(bsrc, 0, lds + CF::BM * BKF);
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
  __syncthreads();
  if (KT > 1) {
    dma_issue<CF::A_ISSUE, CF::NW>(asrc, BKF, lds + CF::STAGE);
    dma_issue<CF::B_ISSUE, CF::NW>(bsrc, BKF, lds + CF::STAGE + CF::BM * BKF);
  }
  pipe_load(f0, addr[0]);
  pipe_step(acc, f0, f1, addr[1]);
  pipe_step(acc, f1, f0, addr[2]);
  pipe_step(acc, f0, f1, addr[3]);
  // f1 holds the fragments of the last step of tile kt - 1
  for (int kt = 1; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this thread's copies of tile kt landed
    __syncthreads();  // everyone's landed, and everyone is done with tile kt-1's stage
    if (kt + 1 < KT) {
      uint16_t* nxt = lds + ((kt + 1) & 1) * CF::STAGE;
      dma_issue<CF::A_ISSUE, CF::NW>(asrc, (kt + 1) * BKF, nxt);
      dma_issue<CF::B_ISSUE, CF::NW>(bsrc, (kt + 1) * BKF, nxt + CF::BM * BKF);
    }
    const uint32_t so = static_cast<uint32_t>(kt & 1) * (CF::STAGE * 2);
    uint32_t a0[6], a1[6], a2[6], a3[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      a0[q] = addr[0][q] + so;
      a1[q] = addr[1][q] + so;
      a2[q] = addr[2][q] + so;
      a3[q] = addr[3][q] + so;
    }
    pipe_step(acc, f1, f0, a0);  // last step of tile kt - 1, reads of tile kt's first
    pipe_step(acc, f0, f1, a1);
    pipe_step(acc, f1, f0, a2);
    pipe_step(acc, f0, f1, a3);
  }
  pipe_last(acc, f1);
  // MFMA results, then VALU reads of them (outside asm): the reads cannot move
  // above the wait, which has the accumulators as operands
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]),
                 "+v"(acc[1][0]), "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3]));
  __syncthreads();  // operand stages are free for the epilogue
}

// ---- [K][N] operand through LDS as stored, read with the gfx950 transpose load
// The tile holds BKF rows (k) of BN columns (n), N-contiguous, in 32-byte
// chunks; chunk c of row k sits at position c ^ tswz(k), so the 4 rows x 32 B
// one 16-lane group reads, and the groups serviced together, hit distinct banks.
__device__ __forceinline__ int tswz(int k) { return (k & 3) ^ ((k >> 1) & 4); }

template <int BN>
__device__ __forceinline__ int nofs(int k, int n) {  // element offset of (k, n) in the tile
  return k * BN + ((((n >> 4) ^ tswz(k)) & (BN / 16 - 1)) << 4) + (n & 15);
}

// DMA sources: instruction i of wave w fills 1 KB = 1024 / (2 BN) rows.
template <int BN, int ISSUE, int NW>
__device__ __forceinline__ void dma_sources_kn(const uint16_t* __restrict__ base, int64_t ld, int N,
                                               int n0, const uint16_t* (&src)[ISSUE]) {
  constexpr int ROWS_PER_KB = 512 / BN;  // rows of BN bf16 in 1 KB
  const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ISSUE; ++i) {
    const int blk = wave + NW * i;
    const int lane_bytes = lane * 16;
    const int k = blk * ROWS_PER_KB + lane_bytes / (BN * 2);
    const int pos = (lane_bytes % (BN * 2)) / 32;  // 32-byte chunk position in the row
    const int half = (lane_bytes / 16) & 1;
    const int c = (pos ^ tswz(k)) & (BN / 16 - 1);
    const int gn = min(n0 + c * 16 + half * 8, N - 8);
    src[i] = base + static_cast<int64_t>(k) * ld + gn;
  }
}

template <int ISSUE, int NW>
__device__ __forceinline__ void dma_issue_kn(const uint16_t* const* src, int64_t k0_times_ld,
                                             uint16_t* tile) {
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ISSUE; ++i)
    __builtin_amdgcn_global_load_lds(src[i] + k0_times_ld, tile + (wave + NW * i) * 512, 16, 0, 0);
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;

// B fragment (16 columns starting at nb, k = kb .. kb+7 per lane group) by two
// transpose loads: lane L of a 16-lane group points at row kb + L/4, columns
// nb + 4 (L%4); the load returns rows kb..kb+3 of column nb + L.
template <int BN>
__device__ __forceinline__ bf16x8_t tr_fragment(const uint16_t* tile, int kb, int nb) {
  const int L = lane_id() & 15;
  typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
  const uint16_t* p0 = tile + nofs<BN>(kb + L / 4, nb + 4 * (L & 3));
  const uint16_t* p1 = tile + nofs<BN>(kb + 4 + L / 4, nb + 4 * (L & 3));
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4*)((__attribute__((address_space(3))) uint16_t*)(p0)));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_v4*)((__attribute__((address_space(3))) uint16_t*)(p1)));
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// C[BM x BN] = A[m0.., :] * B[:, n0..] with A [M][K] K-major and B [K][N]
// N-major, both copied by DMA.  K % 64 == 0.
template <class CF>
__device__ __forceinline__ void mainloop_kn(const uint16_t* __restrict__ A, int64_t lda, int M,
                                            int m0, const uint16_t* __restrict__ B, int64_t ldb,
                                            int N, int n0, int K, uint16_t* lds,
                                            f32x4_t (&acc)[CF::FM][CF::FN]) {
  constexpr int B_ISSUE = CF::BN * BKF / 512 / CF::NW;  // 1 KB DMA blocks per thread
  static_assert(B_ISSUE * 512 * CF::NW == CF::BN * BKF, "B tile splits into whole 1 KB blocks");
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int j = 0; j < CF::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint16_t* asrc[CF::A_ISSUE];
  const uint16_t* bsrc[B_ISSUE];
  dma_sources<CF::A_ISSUE, CF::NW, true>(A, lda, M, m0, asrc);
  dma_sources_kn<CF::BN, B_ISSUE, CF::NW>(B, ldb, N, n0, bsrc);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  const int KT = K / BKF;
  dma_issue<CF::A_ISSUE, CF::NW>(asrc, 0, lds);
  dma_issue_kn<B_ISSUE, CF::NW>(bsrc, 0, lds + CF::BM * BKF);
  for (int kt = 0; kt < KT; ++kt) {
    uint16_t* cur = lds + (kt & 1) * CF::STAGE;
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    __syncthreads();
    if (kt + 1 < KT) {
      uint16_t* nxt = lds + ((kt + 1) & 1) * CF::STAGE;
      dma_issue<CF::A_ISSUE, CF::NW>(asrc, (kt + 1) * BKF, nxt);
      dma_issue_kn<B_ISSUE, CF::NW>(bsrc, static_cast<int64_t>(kt + 1) * BKF * ldb,
                                    nxt + CF::BM * BKF);
    }
    const uint16_t* sA = cur;
    const uint16_t* sB = cur + CF::BM * BKF;
#pragma unroll
    for (int ks = 0; ks < BKF / 32; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
      bf16x8_t a[CF::FM], b[CF::FN];
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(sA + tofs16(wm * CF::WTM + i * 16 + (lane & 15), kc));
#pragma unroll
      for (int j = 0; j < CF::FN; ++j)
        b[j] = tr_fragment<CF::BN>(sB, ks * 32 + (lane >> 4) * 8, wn * CF::WTN + j * 16);
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int j = 0; j < CF::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();
}

// Block index -> (m0, n0): blocks are dealt round-robin to the 8 XCDs, so the
// grid is renumbered to give each XCD a contiguous run of tiles, walked in
// groups of GROUP_M row blocks so concurrently running tiles share operands
// in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int m_blocks, int n_blocks, int BM, int BN, int& m0,
                                            int& n0) {
  const int G = m_blocks * n_blocks;
  const int b = blockIdx.x;
  int L = b;
  if (G % 8 == 0) L = (b % 8) * (G / 8) + b / 8;
  const int per_group = GROUP_M * n_blocks;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(GROUP_M, m_blocks - first_m);
  const int in = L - g * per_group;
  m0 = (first_m + in % gm) * BM;
  n0 = (in / gm) * BN;
}

}  // namespace fast

// ---------------------------------------------------------------- G1 kernel
// Epilogue of G1: h = ReLU(acc + b) rounded to bf16 is staged through LDS in
// `passes` rounds of BM/passes rows (all rows at once when the staging area
// holds the whole block, so no accumulator stays live while packing), then
// every (row, tile) of the staged rows is packed by one wave.
template <int BM, int BN, int WAVES_M, int WAVES_N, int WTM, int WTN, int FM, int FN, int NT,
          int PASSES>
__device__ __forceinline__ void up_pack_epilogue(
    const f32x4_t (&acc)[FM][FN], uint16_t* __restrict__ stage, const float* __restrict__ bias,
    int m0, int n0, int M, int N, int T, int C, int nt, uint16_t* __restrict__ vals,
    uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt, uint8_t* __restrict__ flags,
    uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  static_assert(WAVES_M % PASSES == 0, "whole wave rows per pass");
  constexpr int LDS_ST = BN + 8;                   // staging pitch (elements)
  constexpr int ROWS = BM / PASSES;                // rows staged per pass
  constexpr int WM_PER_PASS = WAVES_M / PASSES;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tiles_per_block = BN / T;
#pragma unroll 1
  for (int p = 0; p < PASSES; ++p) {
    __syncthreads();
    if (wm / WM_PER_PASS == p) {
      const int rofs = (wm % WM_PER_PASS) * WTM;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn * WTN + j * 16 + (lane & 15);
        const float bj = n0 + col < N ? bias[n0 + col] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rofs + i * 16 + (lane >> 4) * 4 + r;
            const float z = acc[i][j][r] + bj;
            const float h = z > 0.f ? z : 0.f;  // ReLU; inactive units are +0.0
            stage[row * LDS_ST + col] = ElemTraits<uint16_t>::from_f32(h);
          }
      }
    }
    __syncthreads();
    const int rbase = m0 + p * ROWS;
    for (int q = wave; q < ROWS * tiles_per_block; q += NT / kWave) {
      const int row = q / tiles_per_block;
      const int tt = q % tiles_per_block;
      const int n = rbase + row;
      const int col0 = n0 + tt * T;
      if (n >= M || col0 >= N) continue;
      const int64_t slot = static_cast<int64_t>(n) * nt + col0 / T;
      pack_tile_from<uint16_t>(stage + row * LDS_ST + tt * T, T, C, vals + slot * C, idx + slot * C,
                               cnt + slot, flags + slot,
                               spill ? spill + static_cast<int64_t>(n) * N + col0 : nullptr);
    }
    if (hdebug != nullptr) {
      for (int v = threadIdx.x; v < ROWS * (BN / 8); v += NT) {
        const int row = v / (BN / 8);
        const int cv = v % (BN / 8);
        const int n = rbase + row;
        const int col = n0 + cv * 8;
        if (n < M && col < N)
          *reinterpret_cast<uint4*>(hdebug + static_cast<int64_t>(n) * N + col) =
              *reinterpret_cast<const uint4*>(stage + row * LDS_ST + cv * 8);
      }
    }
  }
}

// Generic G1 (any K % 8 == 0): register-staged operands.
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(kThreads) void up_pack_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up_t,
    const float* __restrict__ bias, int M, int N, int K, int T, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  typedef Tile<BM, BN, WAVES_M, WAVES_N> TL;
  static_assert(TL::WTM * (BN + 8) <= TL::LDS_ELEMS, "staging fits in the operand buffers");
  __shared__ __attribute__((aligned(16))) uint16_t lds[TL::LDS_ELEMS];
  const int n_blocks = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / n_blocks) * BM;
  const int n0 = (blockIdx.x % n_blocks) * BN;
  f32x4_t acc[TL::FM][TL::FN];
  mfma_mainloop<BM, BN, WAVES_M, WAVES_N, true>(x, K, M, m0, w_up_t, K, N, n0, K, lds,
                                                lds + BM * LDK, acc);
  up_pack_epilogue<BM, BN, WAVES_M, WAVES_N, TL::WTM, TL::WTN, TL::FM, TL::FN, kThreads, WAVES_M>(
      acc, lds, bias, m0, n0, M, N, T, C, nt, vals, idx, cnt, flags, spill, hdebug);
}

// Epilogue of the fast G1, straight from the 32x32 MFMA accumulators (no
// staging of h).  In that layout register r of lane l holds row
// (r/4)*8 + (l/32)*4 + r%4 and column l%32 of a 32x32 block, so one ballot per
// (block, register) yields, in each 32-bit half, the non-zero pattern of 32
// consecutive columns of one row.  A wave owns 64 columns (a "segment") of
// 128 rows; a tile of width T spans T/64 segments of adjacent waves:
//   1. h = ReLU(acc + b) rounded to bf16, in place;
//   2. each wave counts the non-zeros of each of its row segments and posts
//      the counts to LDS (one byte per (row, segment));
//   3. after a barrier every lane knows, for its row, the tile's total and the
//      non-zeros in the segments to its left, so each non-zero element knows
//      its slot (column order) and is stored there directly; the tile's first
//      wave writes the count, the overflow flag and the padding slots; a tile
//      over capacity spills its raw h instead.
// When a block's slots of one row fit in 64 (tiles per block x C <= 64), the
// slots, counts and flags are assembled in LDS (zero-filled, so padding needs
// no stores) and copied out with coalesced stores; otherwise each slot is
// stored to global memory where it is found.
constexpr int kStagedSlots = 64;

template <class CF, bool STAGED>
__device__ __forceinline__ void up_pack_epilogue32(
    const fast::f32x16_t (&acc)[CF::WTM / 32][CF::WTN / 32], uint8_t* __restrict__ lds,
    const float* __restrict__ bias, int m0, int n0, int M, int N, int T, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  constexpr int FM = CF::WTM / 32, FN = CF::WTN / 32, BM = CF::BM;
  constexpr int SPW = CF::WTN / 64;  // 64-column segments per wave
  static_assert(CF::WTN % 64 == 0 && CF::BN / 64 <= 4, "whole segments, at most 4 per block row");
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  // LDS: per-(row, segment) counts, then (staged) slot values, indices, counts, flags
  uint8_t* seg = lds;                                            // [BM][4]
  uint16_t* sv = reinterpret_cast<uint16_t*>(lds + BM * 4);      // [BM][kStagedSlots]
  uint8_t* si = lds + BM * 4 + BM * kStagedSlots * 2;            // [BM][kStagedSlots]
  uint8_t* sc = si + BM * kStagedSlots;                          // [BM][4]
  uint8_t* sf = sc + BM * 4;                                     // [BM][4]
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  const int hh = lane >> 5, c = lane & 31;
  const int spt = T / 64;  // segments per tile
  const uint32_t below = (1u << c) - 1u;
  // per segment sj of this wave (block segment sg = wn * SPW + sj)
  int seg_col[SPW], first[SPW], t[SPW], tb[SPW];
  bool seg_ok[SPW];
  uint32_t tile_mask[SPW], left_mask[SPW];
#pragma unroll
  for (int sj = 0; sj < SPW; ++sj) {
    const int sg = wn * SPW + sj;
    seg_col[sj] = n0 + sg * 64;   // first column of the segment
    seg_ok[sj] = seg_col[sj] < N;  // segments (and tiles) are all-in or all-out
    first[sj] = sg & ~(spt - 1);   // first segment of the segment's tile
    t[sj] = seg_col[sj] / T;       // global tile index
    tb[sj] = (sg * 64) / T;        // tile index inside the block
    // byte masks selecting the tile's segments, and those left of this one
    tile_mask[sj] = (spt == 4 ? 0x01010101u : spt == 2 ? 0x0101u : 0x01u) << (8 * first[sj]);
    const int nleft = sg - first[sj];
    left_mask[sj] = nleft == 0 ? 0u : (0x01010101u >> (8 * (4 - nleft))) << (8 * first[sj]);
  }
  const int tpb = CF::BN / T;  // tiles per block
  if constexpr (STAGED) {
    for (int e = threadIdx.x; e < BM * kStagedSlots / 2; e += CF::NT) {
      reinterpret_cast<uint32_t*>(sv)[e] = 0u;
      if (e < BM * kStagedSlots / 4) reinterpret_cast<uint32_t*>(si)[e] = 0u;
    }
  }
  float bj[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * CF::WTN + j * 32 + c;
    bj[j] = col < N ? bias[col] : 0.f;
  }
  // One 32-row block of the wave's rows; called with constant i below, so the
  // accumulators are only ever indexed statically (no scratch copy).
  auto block = [&](const int i, const fast::f32x16_t (&ai)[FN]) __attribute__((always_inline)) {
    // 1. h = ReLU(acc + b) as bf16 (+0.0 when off), two rows per register, RNE
    uint32_t hp[FN][8];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float z0 = ai[j][r] + bj[j], z1 = ai[j][r + 1] + bj[j];
        const f32x2_t z = {z0 > 0.f ? z0 : 0.f, z1 > 0.f ? z1 : 0.f};
        hp[j][r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(z, bf16x2_t));
      }
    auto hv = [&](int j, int r) -> uint32_t {
      return (r & 1) ? (hp[j][r / 2] >> 16) : (hp[j][r / 2] & 0xffffu);
    };
    auto half = [&](uint64_t m) -> uint32_t {
      return hh ? static_cast<uint32_t>(m >> 32) : static_cast<uint32_t>(m);
    };
    // 2. non-zero count per (row, segment) to LDS: the two ballots of a
    // segment's 32-column halves, counted per 32-lane half of the wave (one
    // row each); lane 0 posts the first row, lane 32 the second
    const int rl0 = wm * CF::WTM + i * 32 + hh * 4;  // row of register r = rl0 + (r/4)*8 + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int sj = 0; sj < SPW; ++sj) {
        const uint64_t b0 = wave_ballot(hv(2 * sj, r) != 0u);
        const uint64_t b1 = wave_ballot(hv(2 * sj + 1, r) != 0u);
        const int lo = __popc(static_cast<uint32_t>(b0)) + __popc(static_cast<uint32_t>(b1));
        const int hi = __popc(static_cast<uint32_t>(b0 >> 32)) + __popc(static_cast<uint32_t>(b1 >> 32));
        if (c == 0)
          seg[(rl0 + (r >> 2) * 8 + (r & 3)) * 4 + wn * SPW + sj] = static_cast<uint8_t>(hh ? hi : lo);
      }
    __syncthreads();
    // 3. slots, metadata, spill (the ballots are taken again: cheaper than
    // keeping them live across the barrier)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = rl0 + (r >> 2) * 8 + (r & 3);
      const int n = m0 + rl;
      const uint32_t counts = *reinterpret_cast<const uint32_t*>(seg + rl * 4);
#pragma unroll
      for (int sj = 0; sj < SPW; ++sj) {
        const int total = static_cast<int>(__builtin_amdgcn_udot4(counts, tile_mask[sj], 0u, false));
        const int left = static_cast<int>(__builtin_amdgcn_udot4(counts, left_mask[sj], 0u, false));
        const bool fits = total <= C;
        const bool row_ok = seg_ok[sj] && n < M;
        const int64_t slot0 = (static_cast<int64_t>(n) * nt + t[sj]) * C;
        const uint32_t cm0 = half(wave_ballot(hv(2 * sj, r) != 0u));
        const uint32_t cm1 = half(wave_ballot(hv(2 * sj + 1, r) != 0u));
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int j = 2 * sj + h2;
          const uint32_t v = hv(j, r);
          const int col = seg_col[sj] + h2 * 32 + c;
          if (row_ok && v != 0u && fits) {
            const int pos = left + (h2 ? __popc(cm0) : 0) + __popc((h2 ? cm1 : cm0) & below);
            if constexpr (STAGED) {
              sv[rl * kStagedSlots + tb[sj] * C + pos] = static_cast<uint16_t>(v);
              si[rl * kStagedSlots + tb[sj] * C + pos] = static_cast<uint8_t>(col - t[sj] * T);
            } else {
              vals[slot0 + pos] = static_cast<uint16_t>(v);
              idx[slot0 + pos] = static_cast<uint8_t>(col - t[sj] * T);
            }
          }
          if (row_ok && !fits && spill != nullptr)
            spill[static_cast<int64_t>(n) * N + col] = static_cast<uint16_t>(v);
          if (row_ok && hdebug != nullptr)
            hdebug[static_cast<int64_t>(n) * N + col] = static_cast<uint16_t>(v);
        }
        if (row_ok && wn * SPW + sj == first[sj]) {
          if constexpr (STAGED) {
            if (c == 0) {
              sc[rl * 4 + tb[sj]] = static_cast<uint8_t>(fits ? total : 0);
              sf[rl * 4 + tb[sj]] = static_cast<uint8_t>(fits ? 0 : 1);
            }
          } else {
            if (c == 0) {
              cnt[static_cast<int64_t>(n) * nt + t[sj]] = static_cast<uint8_t>(fits ? total : 0);
              flags[static_cast<int64_t>(n) * nt + t[sj]] = static_cast<uint8_t>(fits ? 0 : 1);
            }
            if (fits)
              for (int sl = total + c; sl < C; sl += 32) {
                vals[slot0 + sl] = 0;
                idx[slot0 + sl] = 0;
              }
          }
        }
      }
    }
  };
  static_assert(FM <= 4, "up to four 32-row blocks per wave");
  block(0, acc[0]);
  if constexpr (FM > 1) block(1, acc[1]);
  if constexpr (FM > 2) block(2, acc[2]);
  if constexpr (FM > 3) block(3, acc[3]);
  if constexpr (STAGED) {
    __syncthreads();
    // copy the block's slots out: each row owns one contiguous run per array
    const int t0 = n0 / T;
    const int tv = min(tpb, nt - t0);  // tiles of the block inside d_ff
    const int run = tv * C;
    for (int e = threadIdx.x; e < BM * run; e += CF::NT) {
      const int rl = e / run, k = e - (e / run) * run;
      const int n = m0 + rl;
      if (n < M) {
        const int64_t g = (static_cast<int64_t>(n) * nt + t0) * C + k;
        vals[g] = sv[rl * kStagedSlots + k];
        idx[g] = si[rl * kStagedSlots + k];
      }
    }
    for (int e = threadIdx.x; e < BM * tv; e += CF::NT) {
      const int rl = e / tv, k = e - (e / tv) * tv;
      const int n = m0 + rl;
      if (n < M) {
        cnt[static_cast<int64_t>(n) * nt + t0 + k] = sc[rl * 4 + k];
        flags[static_cast<int64_t>(n) * nt + t0 + k] = sf[rl * 4 + k];
      }
    }
  }
}

// Fast G1 (K % 64 == 0): 32x32x16 MFMA mainloop, pack straight from registers.
template <class CF>
__global__ __launch_bounds__(CF::NT) void up_pack_bf16_fast(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up_t,
    const float* __restrict__ bias, int M, int N, int K, int T, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE];
  int m0, n0;
  fast::tile_coords<4>((M + CF::BM - 1) / CF::BM, (N + CF::BN - 1) / CF::BN, CF::BM, CF::BN, m0, n0);
  fast::f32x16_t acc[CF::WTM / 32][CF::WTN / 32];
  fast::mainloop32<CF>(x, K, M, m0, w_up_t, K, N, n0, K, lds, acc);
  if ((CF::BN / T) * C <= kStagedSlots)
    up_pack_epilogue32<CF, true>(acc, reinterpret_cast<uint8_t*>(lds), bias, m0, n0, M, N, T, C,
                                 nt, vals, idx, cnt, flags, spill, hdebug);
  else
    up_pack_epilogue32<CF, false>(acc, reinterpret_cast<uint8_t*>(lds), bias, m0, n0, M, N, T, C,
                                  nt, vals, idx, cnt, flags, spill, hdebug);
}

// The lowest remaining element of a segment given as its even (bit m: element
// 2 m) and odd (bit m: element 2 m + 1) non-zero masks, which loses that bit.
// Returns 0xfffffffe or more when both masks are empty.
__device__ __forceinline__ uint32_t ffbl64(uint64_t m) {
  // find-first-bit gives 0xffffffff for 0; OR-ing 32 keeps that and adds 32 otherwise
  uint32_t lo, hi;
  asm("v_ffbl_b32 %0, %1" : "=v"(lo) : "v"(static_cast<uint32_t>(m)));
  asm("v_ffbl_b32 %0, %1" : "=v"(hi) : "v"(static_cast<uint32_t>(m >> 32)));
  return min(lo, hi | 32u);
}

// Word w of ev / od covers elements [128 w, 128 w + 128).
template <int EW>
__device__ __forceinline__ uint32_t lowest_element(uint64_t (&ev)[EW], uint64_t (&od)[EW]) {
  uint32_t e = 0xffffffffu;
  int hit = -1;
  bool even = false;
#pragma unroll
  for (int w = 0; w < EW; ++w) {
    const uint32_t e0 = 2u * ffbl64(ev[w]), e1 = 2u * ffbl64(od[w]) + 1u;
    const uint32_t ew = min(e0, e1);
    if (hit < 0 && ew < 0x80000000u) {
      hit = w;
      even = e0 < e1;
      e = ew + 128u * w;
    }
  }
#pragma unroll
  for (int w = 0; w < EW; ++w) {
    if (w == hit) {
      if (even) ev[w] &= ev[w] - 1; else od[w] &= od[w] - 1;
    }
  }
  return e;
}

// dst[0, bytes) = src[0, bytes) in the widest unit that divides both
// addresses and the length (src in LDS).
__device__ __forceinline__ void copy_run(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
                                         int bytes) {
  const uint32_t al = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)) |
                      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(src)) |
                      static_cast<uint32_t>(bytes);
  if ((al & 15u) == 0) {
    for (int o = 0; o < bytes; o += 16)
      *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
  } else if ((al & 7u) == 0) {
    for (int o = 0; o < bytes; o += 8)
      *reinterpret_cast<uint2*>(dst + o) = *reinterpret_cast<const uint2*>(src + o);
  } else if ((al & 3u) == 0) {
    for (int o = 0; o < bytes; o += 4)
      *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
  } else if ((al & 1u) == 0) {
    for (int o = 0; o < bytes; o += 2)
      *reinterpret_cast<uint16_t*>(dst + o) = *reinterpret_cast<const uint16_t*>(src + o);
  } else {
    for (int o = 0; o < bytes; ++o) dst[o] = src[o];
  }
}

// ReLU of an accumulator: v_max_f32 against 0 gives 0 for a negative, -0 or
// NaN z (MFMA results are never signalling NaNs), as z > 0 ? z : 0 does.
__device__ __forceinline__ float relu_acc(float z) {
  float o;
  asm("v_max_f32 %0, 0, %1" : "=v"(o) : "v"(z));
  return o;
}

// 16-byte chunk swizzle of the LDS h tile: rows 4 q .. 4 q + 3 share
// bitrev4(q & 15), so a lane's 4 rows of one MFMA register group sit at fixed
// offsets, the two row halves of a write (rows 4 apart) land 8 chunks apart,
// and 16 rows 4 apart read by 16 lanes hit 16 distinct chunk columns.
__device__ __forceinline__ int hswz(int row) {
  const int q = (row >> 2) & 15;
  return ((q & 1) << 3) | ((q & 2) << 1) | ((q & 4) >> 1) | ((q & 8) >> 3);
}

// Pack epilogue through LDS for 256-column blocks.  The block's h (ReLU, then
// bf16) goes to LDS as a [BM][256] tile of 512-byte rows with hswz-swizzled
// 16-byte chunks.  Then each thread packs whole (row, tile) segments (per
// wave 64 rows of one tile, rows 4 apart in each 16-lane group): a non-zero
// mask over the segment (two elements per 32-bit word test), its count, and
// the first non-zeros in ascending column order, stored straight to the TwELL
// arrays; an overflowing segment gets count 0, flag 1, padding slots, and its
// raw h in the spill area.  CMAX bounds C (slots are unrolled CMAX times,
// those past C predicated off).
template <class CF, int T, int CMAX, bool HDEBUG>
__device__ __forceinline__ void up_pack_epilogue_lds(
    const fast::f32x16_t (&acc)[CF::WTM / 32][CF::WTN / 32], uint8_t* __restrict__ lds,
    int m0, int n0, int M, int N, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  constexpr int FM = CF::WTM / 32, FN = CF::WTN / 32, BM = CF::BM, BN = CF::BN;
  static_assert(BN == 256 && CF::WTM == 64 && CF::WTN == 128, "512-byte LDS rows, 64 x 128 waves");
  static_assert(T == 64 || T == 128 || T == 256, "whole 16-byte chunks, whole tiles per block");
  static_assert(CMAX % 4 == 0, "whole words of slots");
  constexpr int ROWB = BN * 2;   // bytes per LDS row
  constexpr int CH = T / 8;      // 16-byte chunks per segment
  constexpr int MW = T / 32;     // mask words per segment
  constexpr int TPB = BN / T;    // segments per row of the block
  // C <= 8: the slots are staged in LDS after the h tile and stored by rows
  constexpr bool STAGED = CMAX <= 8;
  static_assert(!STAGED || CF::NT == 2 * BM, "two threads per row for the stores");
  uint16_t* sv = reinterpret_cast<uint16_t*>(lds + BM * ROWB);  // [BM][TPB * C]
  uint8_t* si = reinterpret_cast<uint8_t*>(sv + BM * TPB * C);  // [BM][TPB * C]
  uint8_t* sc = si + BM * TPB * C;                               // [BM][TPB]
  uint8_t* sf = sc + BM * TPB;                                   // [BM][TPB]
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  const int hh = lane >> 5, c = lane & 31;
  {
    // register 4 p + s of block (i, j) is row wm 64 + i 32 + p 8 + 4 hh + s,
    // column wn 128 + j 32 + c; its chunk is (wn 16 + j 4 + c / 8) ^ hswz(row)
    // = lanepart ^ cp(i, j, p), with hswz(row) = 8 hh ^ cp-bits of (i, p)
    const uint32_t lanepart = static_cast<uint32_t>(wn * 16 + ((c >> 3) ^ (hh << 3))) << 4;
    uint8_t* lb = lds + (wm * 64 + 4 * hh) * ROWB + (c & 7) * 2;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t cp = static_cast<uint32_t>(((j ^ (p & 1)) << 2) ^ ((p >> 1) << 1) ^ i) << 4;
          uint8_t* a = lb + (lanepart ^ cp) + (i * 32 + p * 8) * ROWB;
#pragma unroll
          for (int s = 0; s < 4; s += 2) {
            const f32x2_t z = {relu_acc(acc[i][j][4 * p + s]), relu_acc(acc[i][j][4 * p + s + 1])};
            const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(z, bf16x2_t));
            *reinterpret_cast<uint16_t*>(a + s * ROWB) = static_cast<uint16_t>(hp);
            *reinterpret_cast<uint16_t*>(a + (s + 1) * ROWB) = static_cast<uint16_t>(hp >> 16);
          }
        }
  }
  __syncthreads();
  const int t0 = n0 / T;
  for (int it = threadIdx.x; it < BM * TPB; it += CF::NT) {
    const int tl = it / BM, within = it % BM;
    const int r = (within & ~63) + 4 * (within & 15) + ((within >> 4) & 3);
    const int n = m0 + r, t = t0 + tl;
    if (n >= M || t >= nt) continue;
    const uint8_t* rowp = lds + r * ROWB;
    const int sw = hswz(r);
    uint32_t mask[MW];
#pragma unroll
    for (int w = 0; w < MW; ++w) mask[w] = 0u;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const uint4 d = *reinterpret_cast<const uint4*>(rowp + (((tl * CH + k) ^ sw) << 4));
      if constexpr (HDEBUG)
        *reinterpret_cast<uint4*>(hdebug + static_cast<int64_t>(n) * N + t * T + k * 8) = d;
      const uint32_t dd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // bit 0 / 16 set when the low / high bf16 is non-zero (sign ignored)
        uint32_t f;
        asm("v_pk_min_u16 %0, %1, %2" : "=v"(f) : "v"(dd[q] & 0x7fff7fffu), "s"(0x00010001u));
        mask[k / 4] |= f << ((k % 4) * 4 + q);
      }
    }
    int count = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) count += __popc(mask[w]);
    const bool fits = count <= C;
    // even / odd elements of the segment: bit m of ev / od (over its 64-bit
    // words) is element 2 m / 2 m + 1
    constexpr int EW = (T + 127) / 128;
    uint64_t ev[EW], od[EW];
#pragma unroll
    for (int w = 0; w < EW; ++w) ev[w] = od[w] = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) {
      ev[w / 4] |= static_cast<uint64_t>(mask[w] & 0xffffu) << (16 * (w % 4));
      od[w / 4] |= static_cast<uint64_t>(mask[w] >> 16) << (16 * (w % 4));
    }
    if (!fits) {
#pragma unroll
      for (int w = 0; w < EW; ++w) ev[w] = od[w] = 0;
    }
    uint32_t vp[CMAX / 2], ip[CMAX / 4];
#pragma unroll
    for (int k = 0; k < CMAX / 2; ++k) vp[k] = 0u;
#pragma unroll
    for (int k = 0; k < CMAX / 4; ++k) ip[k] = 0u;
#pragma unroll
    for (int k = 0; k < CMAX; ++k) {
      if (k >= C) break;
      const uint32_t e = lowest_element<EW>(ev, od);  // >= 2^31 when none is left
      if (e < 0x80000000u) {
        const int lc = tl * T + static_cast<int>(e);  // column inside the block
        const uint32_t v = *reinterpret_cast<const uint16_t*>(
            rowp + (((lc >> 3) ^ sw) << 4) + ((lc & 7) << 1));
        vp[k / 2] |= v << (16 * (k % 2));
        ip[k / 4] |= e << (8 * (k % 4));
      }
    }
    if (!fits && spill != nullptr) {
#pragma unroll
      for (int k = 0; k < CH; ++k)
        *reinterpret_cast<uint4*>(spill + static_cast<int64_t>(n) * N + t * T + k * 8) =
            *reinterpret_cast<const uint4*>(rowp + (((tl * CH + k) ^ sw) << 4));
    }
    if constexpr (STAGED) {
      // the row's run of TPB * C slots in LDS, stored by rows below
      const int o = r * TPB * C + tl * C;
      if ((C & 1) == 0) {
#pragma unroll
        for (int k = 0; k < CMAX / 2; ++k)
          if (2 * k < C) reinterpret_cast<uint32_t*>(sv + o)[k] = vp[k];
      } else {
#pragma unroll
        for (int k = 0; k < CMAX; ++k)
          if (k < C) sv[o + k] = static_cast<uint16_t>(vp[k / 2] >> (16 * (k % 2)));
      }
      if ((C & 3) == 0) {
#pragma unroll
        for (int k = 0; k < CMAX / 4; ++k)
          if (4 * k < C) reinterpret_cast<uint32_t*>(si + o)[k] = ip[k];
      } else {
#pragma unroll
        for (int k = 0; k < CMAX; ++k)
          if (k < C) si[o + k] = static_cast<uint8_t>(ip[k / 4] >> (8 * (k % 4)));
      }
      sc[r * TPB + tl] = static_cast<uint8_t>(fits ? count : 0);
      sf[r * TPB + tl] = fits ? 0 : 1;
    } else {
      const int64_t g = (static_cast<int64_t>(n) * nt + t) * C;
      if ((C & 1) == 0) {
#pragma unroll
        for (int k = 0; k < CMAX / 2; ++k)
          if (2 * k < C) reinterpret_cast<uint32_t*>(vals + g)[k] = vp[k];
      } else {
#pragma unroll
        for (int k = 0; k < CMAX; ++k)
          if (k < C) vals[g + k] = static_cast<uint16_t>(vp[k / 2] >> (16 * (k % 2)));
      }
      if ((C & 3) == 0) {
#pragma unroll
        for (int k = 0; k < CMAX / 4; ++k)
          if (4 * k < C) reinterpret_cast<uint32_t*>(idx + g)[k] = ip[k];
      } else {
#pragma unroll
        for (int k = 0; k < CMAX; ++k)
          if (k < C) idx[g + k] = static_cast<uint8_t>(ip[k / 4] >> (8 * (k % 4)));
      }
      cnt[static_cast<int64_t>(n) * nt + t] = static_cast<uint8_t>(fits ? count : 0);
      flags[static_cast<int64_t>(n) * nt + t] = fits ? 0 : 1;
    }
  }
  if constexpr (STAGED) {
    // one thread per row and array group: a row's runs are contiguous in every array
    __syncthreads();
    const int r = threadIdx.x % BM;
    const int n = m0 + r;
    const int tv = min(TPB, nt - t0);  // tiles of the block inside d_ff
    if (n < M && tv > 0) {
      const int64_t g = static_cast<int64_t>(n) * nt + t0;
      if (threadIdx.x < BM) {
        copy_run(reinterpret_cast<uint8_t*>(vals + g * C),
                 reinterpret_cast<const uint8_t*>(sv + r * TPB * C), tv * C * 2);
      } else {
        copy_run(idx + g * C, si + r * TPB * C, tv * C);
        copy_run(cnt + g, sc + r * TPB, tv);
        copy_run(flags + g, sf + r * TPB, tv);
      }
    }
  }
}

// Fast G1 with waves of 64 x 128 on 256-column blocks, packed through LDS
// (C <= CMAX).
template <class CF, int T, int CMAX, bool HDEBUG>
__global__ __launch_bounds__(CF::NT) void up_pack_bf16_wave(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up_t,
    const float* __restrict__ bias, int M, int N, int K, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  // two operand stages, which the epilogue reuses for the h tile; then, for
  // C <= 8, the staged slots: (2 + 1) bytes per slot and 2 per (row, tile)
  constexpr int STAGED_BYTES = CMAX <= 8 ? CF::BM * (CF::BN / T) * (3 * CMAX + 2) : 0;
  static_assert(2 * CF::STAGE * 2 >= CF::BM * CF::BN * 2, "the h tile fits the stages");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE + STAGED_BYTES / 2];
  int m0, n0;
  fast::tile_coords<4>((M + CF::BM - 1) / CF::BM, (N + CF::BN - 1) / CF::BN, CF::BM, CF::BN, m0, n0);
  fast::f32x16_t acc[CF::WTM / 32][CF::WTN / 32];
  float bj[4];  // z starts at the bias of the lane's column in each 32-column block
  {
    const int wn = (threadIdx.x / kWave) % CF::WAVES_N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * CF::WTN + j * 32 + (lane_id() & 31);
      bj[j] = col < N ? bias[col] : 0.f;
    }
  }
  fast::mainloop32_pipe<CF>(x, K, M, m0, w_up_t, K, N, n0, K, lds, bj, acc);
  up_pack_epilogue_lds<CF, T, CMAX, HDEBUG>(acc, reinterpret_cast<uint8_t*>(lds), m0, n0, M, N, C,
                                            nt, vals, idx, cnt, flags, spill, hdebug);
}

// ---------------------------------------------------------------- G4 kernel
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(kThreads) void fallback_bf16_kernel(
    const uint16_t* __restrict__ dense_values, const int32_t* __restrict__ dense_rows,
    const int32_t* __restrict__ n_dense, int64_t dense_cap, const uint16_t* __restrict__ w_down,
    uint16_t* __restrict__ y, int64_t y_rows, int N, int K) {
  typedef Tile<BM, BN, WAVES_M, WAVES_N> TL;
  __shared__ __attribute__((aligned(16))) uint16_t lds[TL::LDS_ELEMS];
  const int64_t stored = min(static_cast<int64_t>(*n_dense), dense_cap);
  const int M = static_cast<int>(stored);
  const int n_blocks = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / n_blocks) * BM;
  const int n0 = (blockIdx.x % n_blocks) * BN;
  if (m0 >= M) return;  // grid sized for the worst case; surplus blocks leave

  f32x4_t acc[TL::FM][TL::FN];
  mfma_mainloop<BM, BN, WAVES_M, WAVES_N, false>(dense_values, K, M, m0, w_down, N, N, n0, K, lds,
                                                 lds + BM * LDK, acc);
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * TL::WTM + i * 16 + (lane >> 4) * 4 + r;
      if (m >= M) continue;
      const int64_t yrow = dense_rows[m];
      if (yrow < 0 || yrow >= y_rows) continue;  // never write outside y
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int col = n0 + wn * TL::WTN + j * 16 + (lane & 15);
        if (col < N) y[yrow * N + col] = ElemTraits<uint16_t>::from_f32(acc[i][j][r]);
      }
    }
}

// Fast G4 (K = d_ff, a multiple of 64): w_down tiles go to LDS as stored and
// are read with the transpose load.  The grid is sized on the host (the live
// row count stays on the device), so each workgroup first works out the
// split: with L live BM x BN tiles and G workgroups, K is cut into
// S = clamp(G / L, 1, ...) slices, workgroup b taking tile b mod L (so the
// live tiles spread over all XCDs) and slice b / L.  With S = 1 the tile is
// rounded and scattered into y; otherwise each slice stores its fp32 partial
// sums part[slice][m][n] for the live rows and fallback_reduce_kernel adds
// the slices in slice order.  S depends only on the live row count and the
// launch, so both kernels derive the same split, and the sum order is fixed.
constexpr int kFbMaxSlices = 32;

struct FbSplit {
  int live_tiles;
  int slices;
};

__device__ __forceinline__ FbSplit fb_split(int M, int BM, int n_blocks, int grid, int ksteps,
                                            int N, const float* part, int64_t part_elems) {
  FbSplit sp;
  sp.live_tiles = ((M + BM - 1) / BM) * n_blocks;
  int s = sp.live_tiles > 0 ? grid / sp.live_tiles : 1;
  s = min(s, min(ksteps, kFbMaxSlices));
  // the partial sums [s][M][N] must fit the scratch
  if (part == nullptr || M <= 0) s = 1;
  else s = static_cast<int>(min(static_cast<int64_t>(s), part_elems / (static_cast<int64_t>(M) * N)));
  sp.slices = max(s, 1);
  return sp;
}

template <class CF>
__global__ __launch_bounds__(CF::NT) void fallback_bf16_fast(
    const uint16_t* __restrict__ dense_values, const int32_t* __restrict__ dense_rows,
    const int32_t* __restrict__ n_dense, int64_t dense_cap, const uint16_t* __restrict__ w_down,
    uint16_t* __restrict__ y, int64_t y_rows, int N, int K, float* __restrict__ part,
    int64_t part_elems) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE];
  const int M = static_cast<int>(min(static_cast<int64_t>(*n_dense), dense_cap));
  const int n_blocks = (N + CF::BN - 1) / CF::BN;
  const int ksteps = K / fast::BKF;
  const FbSplit sp = fb_split(M, CF::BM, n_blocks, static_cast<int>(gridDim.x), ksteps, N, part,
                              part_elems);
  const int b = blockIdx.x;
  if (M <= 0 || b >= sp.live_tiles * sp.slices) return;  // surplus workgroups leave
  const int tile = b % sp.live_tiles, slice = b / sp.live_tiles;
  const int m0 = (tile / n_blocks) * CF::BM;
  const int n0 = (tile % n_blocks) * CF::BN;
  const int k0 = (slice * ksteps / sp.slices) * fast::BKF;
  const int k1 = ((slice + 1) * ksteps / sp.slices) * fast::BKF;
  f32x4_t acc[CF::FM][CF::FN];
  fast::mainloop_kn<CF>(dense_values + k0, K, M, m0, w_down + static_cast<int64_t>(k0) * N, N, N,
                        n0, k1 - k0, lds, acc);
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  float* dst = part + static_cast<int64_t>(slice) * M * N;
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * CF::WTM + i * 16 + (lane >> 4) * 4 + r;
      if (m >= M) continue;
      if (sp.slices > 1) {
#pragma unroll
        for (int j = 0; j < CF::FN; ++j) {
          const int col = n0 + wn * CF::WTN + j * 16 + (lane & 15);
          if (col < N) dst[static_cast<int64_t>(m) * N + col] = acc[i][j][r];
        }
        continue;
      }
      const int64_t yrow = dense_rows[m];
      if (yrow < 0 || yrow >= y_rows) continue;  // never write outside y
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) {
        const int col = n0 + wn * CF::WTN + j * 16 + (lane & 15);
        if (col < N) y[yrow * N + col] = ElemTraits<uint16_t>::from_f32(acc[i][j][r]);
      }
    }
}

// Sum of the fallback's K slices (when fallback_bf16_fast split K): work
// item i adds 8 consecutive outputs of one live row over the slices in slice
// order, rounds them and stores them to y[dense_rows[m]].  The grid is capped
// and strides over the live rows' items, so a few live rows do not pay for a
// worst-case grid of workgroups that only leave; with S = 1 every workgroup
// leaves at once.
constexpr int kFbReduceThreads = 256;
constexpr int kFbReduceGrid = 1024;

__global__ __launch_bounds__(kFbReduceThreads) void fallback_reduce_kernel(
    const float* __restrict__ part, int64_t part_elems, const int32_t* __restrict__ n_dense,
    int64_t dense_cap, const int32_t* __restrict__ dense_rows, uint16_t* __restrict__ y,
    int64_t y_rows, int N, int K, int BM, int BN, int split_grid) {
  const int M = static_cast<int>(min(static_cast<int64_t>(*n_dense), dense_cap));
  const int n_blocks = (N + BN - 1) / BN;
  const FbSplit sp = fb_split(M, BM, n_blocks, split_grid, K / fast::BKF, N, part, part_elems);
  if (M <= 0 || sp.slices == 1) return;
  const int per_row = N / 8;
  const int64_t items = static_cast<int64_t>(M) * per_row;
  const int64_t slice_stride = static_cast<int64_t>(M) * N;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFbReduceThreads + threadIdx.x; i < items;
       i += static_cast<int64_t>(gridDim.x) * kFbReduceThreads) {
    const int m = static_cast<int>(i / per_row);
    const int c = static_cast<int>(i % per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* src = part + static_cast<int64_t>(m) * N + c;
    auto add = [&](const float4& a, const float4& b) {
      acc[0] += a.x, acc[1] += a.y, acc[2] += a.z, acc[3] += a.w;
      acc[4] += b.x, acc[5] += b.y, acc[6] += b.z, acc[7] += b.w;
    };
    int s = 0;
    // 8 slices' loads in flight at once (many slices come from few live rows)
    for (; s + 8 <= sp.slices; s += 8) {
      float4 a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u] = *reinterpret_cast<const float4*>(src + (s + u) * slice_stride);
        b[u] = *reinterpret_cast<const float4*>(src + (s + u) * slice_stride + 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) add(a[u], b[u]);
    }
    for (; s < sp.slices; ++s)
      add(*reinterpret_cast<const float4*>(src + s * slice_stride),
          *reinterpret_cast<const float4*>(src + s * slice_stride + 4));
    const int64_t yrow = dense_rows[m];
    if (yrow < 0 || yrow >= y_rows) continue;  // never write outside y
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * q])) |
             (static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * q + 1])) << 16);
    *reinterpret_cast<uint4*>(y + yrow * N + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ------------------------------------------------- skinny split-K (bf16, <= 64 rows)
// Workgroup (column block, slice) runs the DMA + MFMA main loop over its K
// slice only and stores fp32 partial sums part[slice][m][n] (row stride mm)
// for the live rows; the slice sums and epilogues are shared with the fp32
// skinny kernels.  A has at most 64 rows, so each weight tile is used for one
// MFMA row block and the pair is bound by streaming the weight from HBM.
template <class CF>
__global__ __launch_bounds__(CF::NT) void skinny_up_partial_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up_t, int M, int N, int K,
    int kw, int mm, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE];
  const int n0 = blockIdx.x * CF::BN, slice = blockIdx.y, kbeg = slice * kw;
  fast::f32x16_t acc[CF::WTM / 32][CF::WTN / 32];
  fast::mainloop32<CF>(x + kbeg, K, M, 0, w_up_t + kbeg, K, N, n0, min(kw, K - kbeg), lds, acc);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  float* dst = part + static_cast<int64_t>(slice) * mm * N;
#pragma unroll
  for (int i = 0; i < CF::WTM / 32; ++i)
#pragma unroll
    for (int j = 0; j < CF::WTN / 32; ++j) {
      const int col = n0 + wn * CF::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * CF::WTM + i * 32 + (r / 4) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M && col < N) dst[static_cast<int64_t>(m) * N + col] = acc[i][j][r];
      }
    }
}

// One (column block, K slice) of the fallback's split-K partial sums.
template <class CF>
__device__ __forceinline__ void skinny_fallback_partial_tile(
    const uint16_t* __restrict__ dense_values, const int32_t* __restrict__ n_dense, int m_cap,
    const uint16_t* __restrict__ w_down, int N, int K, int kw, int mm, float* __restrict__ part,
    int nblk, int slice, uint16_t* lds) {
  const int M = min(*n_dense, m_cap);
  if (M <= 0) return;
  const int n0 = nblk * CF::BN, kbeg = slice * kw;
  f32x4_t acc[CF::FM][CF::FN];
  fast::mainloop_kn<CF>(dense_values + kbeg, K, M, 0, w_down + static_cast<int64_t>(kbeg) * N, N,
                        N, n0, min(kw, K - kbeg), lds, acc);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
  float* dst = part + static_cast<int64_t>(slice) * mm * N;
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = wm * CF::WTM + i * 16 + (lane >> 4) * 4 + r;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) {
        const int col = n0 + wn * CF::WTN + j * 16 + (lane & 15);
        if (col < N) dst[static_cast<int64_t>(m) * N + col] = acc[i][j][r];
      }
    }
}

template <class CF>
__global__ __launch_bounds__(CF::NT) void skinny_fallback_partial_bf16(
    const uint16_t* __restrict__ dense_values, const int32_t* __restrict__ n_dense, int m_cap,
    const uint16_t* __restrict__ w_down, int N, int K, int kw, int mm, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE];
  skinny_fallback_partial_tile<CF>(dense_values, n_dense, m_cap, w_down, N, K, kw, mm, part,
                                   blockIdx.x, blockIdx.y, lds);
}

// The few-row sparse product of the TwELL rows in workgroups [0, sp_blocks)
// (one per (row, XCD column slice); sp_blocks is a multiple of 8, so the XCD
// is the workgroup index mod 8 as in its own kernel), and the fallback's
// split-K partial sums in the workgroups after them.  The two write disjoint
// memory (y of the sparse rows, partial sums), so the sparse gathers run
// inside the fallback's weight stream instead of after it; the sparse
// workgroups come first so they start at once.  Each of the CF::NW waves
// takes 16 / CF::NW of the row's 16 tile ranges in turn, so the row's sum is
// the same bits as with the 16-wave kernel.

template <class CF, int VEC>
__global__ __launch_bounds__(CF::NT) void skinny_fallback_partial_spmm_bf16(
    const uint16_t* __restrict__ dense_values, const int32_t* __restrict__ n_dense, int m_cap,
    const uint16_t* __restrict__ w_down, int N, int K, int kw, int mm, float* __restrict__ part,
    int nb, int sp_blocks, SpmmRows sr, uint16_t* __restrict__ y, int64_t rows_max, int T, int C,
    int nt, int n_slices, int tpw) {
  static_assert(kSplitParts % CF::NW == 0, "whole tile ranges per wave");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * CF::STAGE];
  const int b = blockIdx.x;
  if (b < sp_blocks) {
    spmm_split_rows<VEC, CF::NW, kSplitParts / CF::NW>(
        sr.vals, sr.idx, sr.cnt, sr.rows, sr.n_rows, w_down, y, rows_max, N, T, C, nt, n_slices,
        tpw, reinterpret_cast<uint2*>(lds), b, sp_blocks);
    return;
  }
  const int f = b - sp_blocks;
  skinny_fallback_partial_tile<CF>(dense_values, n_dense, m_cap, w_down, N, K, kw, mm, part,
                                   f % nb, f / nb, lds);
}

// 32 rows x 128 columns (4 waves side by side) or 64 x 128 (2 x 2 waves):
// 40-48 KB of LDS, three workgroups per CU.  The up-projection at up to 32
// rows takes 64-column blocks of 2 waves: twice the blocks, each streaming
// 64 weight rows twice as far (measured 34 against 36.5 us for 16 x 4096 x
// 16384; 32-column blocks of one wave 39, 256-column blocks 43.6).
typedef fast::Cfg<32, 128, 1, 4> SkinnyCfg32;
typedef fast::Cfg<64, 128, 2, 2> SkinnyCfg64;
typedef fast::Cfg<32, 64, 1, 2> SkinnyUpCfg32;
constexpr int kSkinnyTargetBlocks = 768;

template <class CF>
hipError_t skinny_up_bf16(const Geometry& g, const uint16_t* x, const uint16_t* w_up_t,
                          const float* b_up, const PackOut& out, hipStream_t s) {
  const int N = g.d_ff, K = g.d_model;
  const int nb = (N + CF::BN - 1) / CF::BN;
  const SkinnySplit sp = skinny_split(g.n_rows, K, nb, fast::BKF, kSkinnyTargetBlocks);
  skinny_up_partial_bf16<CF><<<dim3(nb, sp.slices), CF::NT, 0, s>>>(
      x, w_up_t, static_cast<int>(g.n_rows), N, K, sp.kw, sp.mm, out.skinny);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_skinny_up_epilogue<uint16_t>(g, sp, out.skinny, b_up, out, s);
}

template <class CF>
hipError_t skinny_fallback_bf16(const Geometry& g, const uint16_t* dense_values,
                                const int32_t* dense_rows, const int32_t* n_dense, int m_cap,
                                const uint16_t* w_down, uint16_t* y, float* part, hipStream_t s) {
  const int N = g.d_model, K = g.d_ff;
  const int nb = (N + CF::BN - 1) / CF::BN;
  const SkinnySplit sp = skinny_split(g.n_rows, K, nb, fast::BKF, kSkinnyTargetBlocks);
  skinny_fallback_partial_bf16<CF><<<dim3(nb, sp.slices), CF::NT, 0, s>>>(
      dense_values, n_dense, m_cap, w_down, N, K, sp.kw, sp.mm, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_skinny_fallback_reduce<uint16_t>(g, sp, part, n_dense, m_cap, dense_rows, y, s);
}

template <class CF>
hipError_t skinny_fallback_spmm_bf16(const Geometry& g, const uint16_t* dense_values,
                                     const int32_t* dense_rows, const int32_t* n_dense, int m_cap,
                                     const uint16_t* w_down, uint16_t* y, float* part,
                                     const SpmmRows& sr, const SpmmSplitPlan& pl, hipStream_t s) {
  const int N = g.d_model, K = g.d_ff;
  const int nb = (N + CF::BN - 1) / CF::BN;
  const SkinnySplit sp = skinny_split(g.n_rows, K, nb, fast::BKF, kSkinnyTargetBlocks);
  const unsigned grid = pl.blocks + static_cast<unsigned>(nb * sp.slices);
  const int sp_blocks = static_cast<int>(pl.blocks);  // 8 x rows per XCD
  if (pl.vec == 8)
    skinny_fallback_partial_spmm_bf16<CF, 8><<<grid, CF::NT, 0, s>>>(
        dense_values, n_dense, m_cap, w_down, N, K, sp.kw, sp.mm, part, nb, sp_blocks, sr, y,
        g.n_rows, g.tile, g.capacity, g.n_tiles, pl.n_slices, pl.tpw);
  else
    skinny_fallback_partial_spmm_bf16<CF, 16><<<grid, CF::NT, 0, s>>>(
        dense_values, n_dense, m_cap, w_down, N, K, sp.kw, sp.mm, part, nb, sp_blocks, sr, y,
        g.n_rows, g.tile, g.capacity, g.n_tiles, pl.n_slices, pl.tpw);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || m_cap == 0) return e;  // no dense row can be stored: nothing to sum
  return launch_skinny_fallback_reduce<uint16_t>(g, sp, part, n_dense, m_cap, dense_rows, y, s);
}

// G1: 256 x 256 blocks, 8 waves of 128 x 64 (2 waves per SIMD hide each
// other's LDS waits; 4 waves of 128 x 128 halve the LDS reads per MFMA but
// measured 1.45x slower at one wave per SIMD).
typedef fast::Cfg<256, 256, 2, 4> BigCfg;
// G1 for T = 64 and 128: the same 256 x 256 block, waves of 64 x 128
typedef fast::Cfg<256, 256, 4, 2> BigCfgW;
typedef fast::Cfg<128, 128, 2, 4> MidCfg;
// workgroups of the 128 x 128 fallback when few tiles are live: two per CU
constexpr int kFbSplitGrid = 512;

}  // namespace

hipError_t launch_up_pack_bf16(const Geometry& g, const uint16_t* x, const uint16_t* w_up_t,
                               const float* b_up, const PackOut& out, hipStream_t s) {
  if (out.skinny != nullptr && g.n_rows > 0 && g.n_rows <= kSkinnyMaxRows && g.d_model % 64 == 0)
    return g.n_rows <= 32 ? skinny_up_bf16<SkinnyUpCfg32>(g, x, w_up_t, b_up, out, s)
                          : skinny_up_bf16<SkinnyCfg64>(g, x, w_up_t, b_up, out, s);
  const int M = static_cast<int>(g.n_rows), N = g.d_ff, K = g.d_model;
  if (M == 0) return hipSuccess;
  auto* vals = static_cast<uint16_t*>(out.vals);
  auto* spill = static_cast<uint16_t*>(out.spill);
  auto* hdbg = static_cast<uint16_t*>(out.h_debug);
  const bool wave_tile = g.tile == 64 || g.tile == 128 || (g.tile == 256 && g.capacity <= 8);
  if (M >= 128 && K % 64 == 0 && wave_tile && N % g.tile == 0 &&
      (BigCfgW::BN / g.tile) * g.capacity <= kStagedSlots) {
    const int blocks =
        ((M + BigCfgW::BM - 1) / BigCfgW::BM) * ((N + BigCfgW::BN - 1) / BigCfgW::BN);
    auto go = [&](auto t, auto dbg) {
      // C <= 8 (always for T = 256): slots staged in LDS; larger C up to the
      // 64 slots of a block row stored per thread
      constexpr int T = decltype(t)::value;
      constexpr int CBIG = T == 256 ? 8 : kStagedSlots / (BigCfgW::BN / T);
      if (g.capacity <= 8)
        up_pack_bf16_wave<BigCfgW, T, 8, decltype(dbg)::value>
            <<<blocks, BigCfgW::NT, 0, s>>>(x, w_up_t, b_up, M, N, K, g.capacity, g.n_tiles,
                                           vals, out.idx, out.cnt, out.flags, spill, hdbg);
      else
        up_pack_bf16_wave<BigCfgW, T, CBIG, decltype(dbg)::value>
            <<<blocks, BigCfgW::NT, 0, s>>>(x, w_up_t, b_up, M, N, K, g.capacity, g.n_tiles,
                                           vals, out.idx, out.cnt, out.flags, spill, hdbg);
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using I256 = std::integral_constant<int, 256>;
    using Y = std::true_type;
    using No = std::false_type;
    if (g.tile == 64) hdbg ? go(I64{}, Y{}) : go(I64{}, No{});
    else if (g.tile == 128) hdbg ? go(I128{}, Y{}) : go(I128{}, No{});
    else hdbg ? go(I256{}, Y{}) : go(I256{}, No{});
  } else if (M >= 128 && K % 64 == 0) {
    const int blocks = ((M + BigCfg::BM - 1) / BigCfg::BM) * ((N + BigCfg::BN - 1) / BigCfg::BN);
    up_pack_bf16_fast<BigCfg><<<blocks, BigCfg::NT, 0, s>>>(
        x, w_up_t, b_up, M, N, K, g.tile, g.capacity, g.n_tiles, vals, out.idx, out.cnt, out.flags,
        spill, hdbg);
  } else if (M >= 128) {
    constexpr int BM = 256, BN = 256;
    const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    up_pack_bf16_kernel<BM, BN, 2, 2><<<blocks, kThreads, 0, s>>>(
        x, w_up_t, b_up, M, N, K, g.tile, g.capacity, g.n_tiles, vals, out.idx, out.cnt, out.flags,
        spill, hdbg);
  } else {
    constexpr int BM = 32, BN = 256;
    const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    up_pack_bf16_kernel<BM, BN, 1, 4><<<blocks, kThreads, 0, s>>>(
        x, w_up_t, b_up, M, N, K, g.tile, g.capacity, g.n_tiles, vals, out.idx, out.cnt, out.flags,
        spill, hdbg);
  }
  return hipGetLastError();
}

hipError_t launch_fallback_bf16(const Geometry& g, const uint16_t* dense_values,
                                const int32_t* dense_rows, const int32_t* n_dense,
                                int64_t dense_cap, const uint16_t* w_down, uint16_t* y,
                                hipStream_t s, float* skinny, float* part, int64_t part_elems) {
  const int64_t worst = dense_cap < g.n_rows ? dense_cap : g.n_rows;
  if (worst <= 0) return hipSuccess;
  if (skinny != nullptr && g.n_rows <= kSkinnyMaxRows && g.d_ff % 64 == 0) {
    const int m_cap = static_cast<int>(worst);
    return g.n_rows <= 32 ? skinny_fallback_bf16<SkinnyCfg32>(g, dense_values, dense_rows, n_dense,
                                                             m_cap, w_down, y, skinny, s)
                          : skinny_fallback_bf16<SkinnyCfg64>(g, dense_values, dense_rows, n_dense,
                                                             m_cap, w_down, y, skinny, s);
  }
  const int N = g.d_model, K = g.d_ff;
  // 256 x 256 tiles when even the worst case has at least 8 waves of them
  // (measured: 10% faster for 12839 x 8192 x 28672, slower at 1.2 waves of tiles)
  const int64_t big_tiles = ((worst + BigCfg::BM - 1) / BigCfg::BM) * (N / BigCfg::BN);
  if (K % 64 == 0 && N % BigCfg::BN == 0 && big_tiles >= 2048) {
    fallback_bf16_fast<BigCfg><<<static_cast<int>(big_tiles), BigCfg::NT, 0, s>>>(
        dense_values, dense_rows, n_dense, dense_cap, w_down, y, g.n_rows, N, K, nullptr, 0);
  } else if (worst >= 128 && K % 64 == 0 && N >= 128 && N % 8 == 0) {
    // the worst case's tiles, and at least two workgroups per CU so that a
    // few live tiles split K
    const int64_t tiles =
        ((worst + MidCfg::BM - 1) / MidCfg::BM) * ((N + MidCfg::BN - 1) / MidCfg::BN);
    const int grid = static_cast<int>(tiles > kFbSplitGrid ? tiles : kFbSplitGrid);
    if (part == nullptr) part_elems = 0;
    fallback_bf16_fast<MidCfg><<<grid, MidCfg::NT, 0, s>>>(
        dense_values, dense_rows, n_dense, dense_cap, w_down, y, g.n_rows, N, K, part, part_elems);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || part == nullptr) return e;
    const int64_t outs = worst * (N / 8);
    const int64_t want = (outs + kFbReduceThreads - 1) / kFbReduceThreads;
    const unsigned rblocks = static_cast<unsigned>(want < kFbReduceGrid ? want : kFbReduceGrid);
    fallback_reduce_kernel<<<rblocks, kFbReduceThreads, 0, s>>>(
        part, part_elems, n_dense, dense_cap, dense_rows, y, g.n_rows, N, K, MidCfg::BM,
        MidCfg::BN, grid);
  } else if (worst >= 128) {
    constexpr int BM = 256, BN = 256;
    const int64_t blocks = ((worst + BM - 1) / BM) * ((N + BN - 1) / BN);
    fallback_bf16_kernel<BM, BN, 2, 2><<<static_cast<int>(blocks), kThreads, 0, s>>>(
        dense_values, dense_rows, n_dense, dense_cap, w_down, y, g.n_rows, N, K);
  } else {
    constexpr int BM = 32, BN = 256;
    const int64_t blocks = ((worst + BM - 1) / BM) * ((N + BN - 1) / BN);
    fallback_bf16_kernel<BM, BN, 1, 4><<<static_cast<int>(blocks), kThreads, 0, s>>>(
        dense_values, dense_rows, n_dense, dense_cap, w_down, y, g.n_rows, N, K);
  }
  return hipGetLastError();
}

bool fallback_takes_spmm(const Geometry& g) {
  if (g.n_rows <= 0 || g.n_rows > kSkinnyMaxRows || g.d_ff % 64 != 0) return false;
  SpmmSplitPlan pl;
  if (!spmm_split_plan(g, 4, kSplitParts / 4, &pl)) return false;
  static_assert(SkinnyCfg32::NW == 4 && SkinnyCfg64::NW == 4, "4 sparse waves per workgroup");
  const size_t lds = 2 * static_cast<size_t>(g.n_rows <= 32 ? SkinnyCfg32::STAGE
                                                             : SkinnyCfg64::STAGE) * 2;
  return pl.lds_bytes <= lds;
}

hipError_t launch_fallback_bf16_with_spmm(const Geometry& g, const uint16_t* dense_values,
                                          const int32_t* dense_rows, const int32_t* n_dense,
                                          int64_t dense_cap, const uint16_t* w_down, uint16_t* y,
                                          hipStream_t s, float* skinny, const SpmmRows& sr) {
  SpmmSplitPlan pl;
  if (skinny == nullptr || !fallback_takes_spmm(g) || !spmm_split_plan(g, 4, kSplitParts / 4, &pl))
    return hipErrorInvalidValue;
  const int64_t worst = dense_cap < g.n_rows ? dense_cap : g.n_rows;
  const int m_cap = static_cast<int>(worst > 0 ? worst : 0);
  return g.n_rows <= 32 ? skinny_fallback_spmm_bf16<SkinnyCfg32>(g, dense_values, dense_rows,
                                                                  n_dense, m_cap, w_down, y,
                                                                  skinny, sr, pl, s)
                        : skinny_fallback_spmm_bf16<SkinnyCfg64>(g, dense_values, dense_rows,
                                                                  n_dense, m_cap, w_down, y,
                                                                  skinny, sr, pl, s);
}

}  // namespace twell
