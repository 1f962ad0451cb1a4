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
#include "common.h"
#include "kernels.h"

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

// ---------------------------------------------------------------- G1 kernel
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(kThreads) void up_pack_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up_t,
    const float* __restrict__ bias, int M, int N, int K, int T, int C, int nt,
    uint16_t* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    uint8_t* __restrict__ flags, uint16_t* __restrict__ spill, uint16_t* __restrict__ hdebug) {
  typedef Tile<BM, BN, WAVES_M, WAVES_N> TL;
  constexpr int LDS_ST = BN + 8;  // staging pitch (elements)
  static_assert(TL::WTM * LDS_ST <= TL::LDS_ELEMS, "staging fits in the operand buffers");
  __shared__ __attribute__((aligned(16))) uint16_t lds[TL::LDS_ELEMS];

  const int n_blocks = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / n_blocks) * BM;
  const int n0 = (blockIdx.x % n_blocks) * BN;

  f32x4_t acc[TL::FM][TL::FN];
  mfma_mainloop<BM, BN, WAVES_M, WAVES_N, true>(x, K, M, m0, w_up_t, K, N, n0, K, lds,
                                                lds + BM * LDK, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  float bj[TL::FN];
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) {
    const int col = n0 + wn * TL::WTN + j * 16 + (lane & 15);
    bj[j] = col < N ? bias[col] : 0.f;
  }
  const int tiles_per_block = BN / T;
  uint16_t* stage = lds;

  for (int p = 0; p < WAVES_M; ++p) {
    __syncthreads();
    if (wm == p) {
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = i * 16 + (lane >> 4) * 4 + r;
            const int col = wn * TL::WTN + j * 16 + (lane & 15);
            const float z = acc[i][j][r] + bj[j];
            const float h = z > 0.f ? z : 0.f;  // ReLU; inactive units are +0.0
            stage[row * LDS_ST + col] = ElemTraits<uint16_t>::from_f32(h);
          }
    }
    __syncthreads();
    const int rbase = m0 + p * TL::WTM;
    for (int q = wave; q < TL::WTM * tiles_per_block; q += kThreads / kWave) {
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
      for (int v = threadIdx.x; v < TL::WTM * (BN / 8); v += kThreads) {
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

}  // namespace

hipError_t launch_up_pack_bf16(const Geometry& g, const uint16_t* x, const uint16_t* w_up_t,
                               const float* b_up, const PackOut& out, hipStream_t s) {
  const int M = static_cast<int>(g.n_rows), N = g.d_ff, K = g.d_model;
  if (M == 0) return hipSuccess;
  auto* vals = static_cast<uint16_t*>(out.vals);
  auto* spill = static_cast<uint16_t*>(out.spill);
  auto* hdbg = static_cast<uint16_t*>(out.h_debug);
  if (M >= 128) {
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
                                hipStream_t s) {
  const int64_t worst = dense_cap < g.n_rows ? dense_cap : g.n_rows;
  if (worst <= 0) return hipSuccess;
  const int N = g.d_model, K = g.d_ff;
  if (worst >= 128) {
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

}  // namespace twell
