// float32 versions of the two dense contractions, on the vector ALU (no
// reduced-precision matrix path): G1 up-projection + bias + ReLU + fused TwELL
// pack, and G4 dense fallback.  These serve float32 layers, which are small
// here; bf16 layers use the MFMA kernels.
//
// Block tile 32 x 256 (rows x columns), 256 threads: thread (tr, tc) owns rows
// tr*4 .. tr*4+3 and columns tc + 32*j (j < 8), K staged through LDS 32 at a time.
#include "common.h"
#include "kernels.h"

namespace twell {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 32, BN = 256, BKF = 32;

// ---------------------------------------------------------------- G1 (fp32)
__global__ __launch_bounds__(kThreads) void up_pack_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w_up_t, const float* __restrict__ bias,
    int M, int N, int K, int T, int C, int nt, float* __restrict__ vals, uint8_t* __restrict__ idx,
    uint8_t* __restrict__ cnt, uint8_t* __restrict__ flags, float* __restrict__ spill,
    float* __restrict__ hdebug) {
  constexpr int LDS_ST = BN + 4;
  constexpr int OPER = (BM + BN) * (BKF + 1);
  constexpr int ELEMS = OPER > BM * LDS_ST ? OPER : BM * LDS_ST;
  __shared__ float lds[ELEMS];
  float* sA = lds;                    // [BM][BKF+1]
  float* sB = lds + BM * (BKF + 1);   // [BN][BKF+1]

  const int n_blocks = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / n_blocks) * BM;
  const int n0 = (blockIdx.x % n_blocks) * BN;
  const int tid = threadIdx.x;
  const int tr = tid / 32, tc = tid % 32;

  float acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[r][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int e = tid; e < BM * BKF; e += kThreads) {
      const int r = e / BKF, kk = e % BKF;
      const int gr = m0 + r, gk = k0 + kk;
      sA[r * (BKF + 1) + kk] = (gr < M && gk < K) ? x[static_cast<int64_t>(gr) * K + gk] : 0.f;
    }
    for (int e = tid; e < BN * BKF; e += kThreads) {
      const int c = e / BKF, kk = e % BKF;
      const int gc = n0 + c, gk = k0 + kk;
      sB[c * (BKF + 1) + kk] = (gc < N && gk < K) ? w_up_t[static_cast<int64_t>(gc) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = sA[(tr * 4 + r) * (BKF + 1) + kk];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = sB[(tc + 32 * j) * (BKF + 1) + kk];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = fmaf(a[r], b[j], acc[r][j]);
    }
    __syncthreads();
  }

  float* stage = lds;  // [BM][LDS_ST]
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = tc + 32 * j;
    const float bj = (n0 + col < N) ? bias[n0 + col] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z = acc[r][j] + bj;
      stage[(tr * 4 + r) * LDS_ST + col] = z > 0.f ? z : 0.f;  // ReLU; inactive -> +0.0
    }
  }
  __syncthreads();
  const int wave = tid / kWave;
  const int tiles_per_block = BN / T;
  for (int q = wave; q < BM * tiles_per_block; q += kThreads / kWave) {
    const int row = q / tiles_per_block;
    const int tt = q % tiles_per_block;
    const int n = m0 + row;
    const int col0 = n0 + tt * T;
    if (n >= M || col0 >= N) continue;
    const int64_t slot = static_cast<int64_t>(n) * nt + col0 / T;
    pack_tile_from<float>(stage + row * LDS_ST + tt * T, T, C, vals + slot * C, idx + slot * C,
                          cnt + slot, flags + slot,
                          spill ? spill + static_cast<int64_t>(n) * N + col0 : nullptr);
  }
  if (hdebug != nullptr) {
    for (int e = tid; e < BM * BN; e += kThreads) {
      const int row = e / BN, col = e % BN;
      if (m0 + row < M && n0 + col < N)
        hdebug[static_cast<int64_t>(m0 + row) * N + n0 + col] = stage[row * LDS_ST + col];
    }
  }
}

// ---------------------------------------------------------------- G4 (fp32)
// y[dense_rows[m]] = dense_values[m] @ w_down; w_down is [K][N] (N contiguous).
__global__ __launch_bounds__(kThreads) void fallback_f32_kernel(
    const float* __restrict__ dense_values, const int32_t* __restrict__ dense_rows,
    const int32_t* __restrict__ n_dense, int64_t dense_cap, const float* __restrict__ w_down,
    float* __restrict__ y, int64_t y_rows, int N, int K) {
  __shared__ float sA[BM * (BKF + 1)];
  __shared__ float sB[BKF * BN];
  const int M = static_cast<int>(min(static_cast<int64_t>(*n_dense), dense_cap));
  const int n_blocks = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / n_blocks) * BM;
  const int n0 = (blockIdx.x % n_blocks) * BN;
  if (m0 >= M) return;
  const int tid = threadIdx.x;
  const int tr = tid / 32, tc = tid % 32;
  float acc[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[r][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int e = tid; e < BM * BKF; e += kThreads) {
      const int r = e / BKF, kk = e % BKF;
      const int gr = m0 + r, gk = k0 + kk;
      sA[r * (BKF + 1) + kk] =
          (gr < M && gk < K) ? dense_values[static_cast<int64_t>(gr) * K + gk] : 0.f;
    }
    for (int e = tid; e < BKF * BN; e += kThreads) {
      const int kk = e / BN, c = e % BN;
      const int gc = n0 + c, gk = k0 + kk;
      sB[kk * BN + c] = (gc < N && gk < K) ? w_down[static_cast<int64_t>(gk) * N + gc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = sA[(tr * 4 + r) * (BKF + 1) + kk];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = sB[kk * BN + tc + 32 * j];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = fmaf(a[r], b[j], acc[r][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + tr * 4 + r;
    if (m >= M) continue;
    const int64_t yrow = dense_rows[m];
    if (yrow < 0 || yrow >= y_rows) continue;  // never write outside y
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = n0 + tc + 32 * j;
      if (col < N) y[yrow * N + col] = acc[r][j];
    }
  }
}

}  // namespace

hipError_t launch_up_pack_f32(const Geometry& g, const float* x, const float* w_up_t,
                              const float* b_up, const PackOut& out, hipStream_t s) {
  if (out.skinny != nullptr && g.n_rows <= kSkinnyMaxRows)
    return launch_skinny_up_pack_f32(g, x, w_up_t, b_up, out, out.skinny, s);
  const int M = static_cast<int>(g.n_rows), N = g.d_ff, K = g.d_model;
  if (M == 0) return hipSuccess;
  const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  up_pack_f32_kernel<<<blocks, kThreads, 0, s>>>(
      x, w_up_t, b_up, M, N, K, g.tile, g.capacity, g.n_tiles, static_cast<float*>(out.vals),
      out.idx, out.cnt, out.flags, static_cast<float*>(out.spill), static_cast<float*>(out.h_debug));
  return hipGetLastError();
}

hipError_t launch_fallback_f32(const Geometry& g, const float* dense_values,
                               const int32_t* dense_rows, const int32_t* n_dense,
                               int64_t dense_cap, const float* w_down, float* y, hipStream_t s,
                               float* skinny) {
  const int64_t worst = dense_cap < g.n_rows ? dense_cap : g.n_rows;
  if (worst <= 0) return hipSuccess;
  if (skinny != nullptr && g.n_rows <= kSkinnyMaxRows)
    return launch_skinny_fallback_f32(g, dense_values, dense_rows, n_dense, dense_cap, w_down, y,
                                      skinny, s);
  const int N = g.d_model, K = g.d_ff;
  const int64_t blocks = ((worst + BM - 1) / BM) * ((N + BN - 1) / BN);
  fallback_f32_kernel<<<static_cast<int>(blocks), kThreads, 0, s>>>(dense_values, dense_rows,
                                                                    n_dense, dense_cap, w_down, y,
                                                                    g.n_rows, N, K);
  return hipGetLastError();
}

}  // namespace twell
