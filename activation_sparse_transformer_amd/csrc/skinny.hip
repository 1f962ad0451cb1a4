// Skinny GEMMs: batches of at most 64 rows (decode-sized) against a large
// weight.  One workgroup per output-column block would leave most CUs idle
// and each one waiting on a long K loop, so K is split: workgroup (nb, slice)
// multiplies all rows of A[:, slice K range] with the matching rows of the
// weight for its column block and stores fp32 partial sums
// part[slice][m][n]; a second kernel adds the slices in slice order and
// applies the epilogue.  The weight is streamed once, so the pair is HBM-bound.
//
// This file holds the fp32 partial kernels (VALU: the A slice in LDS, each
// thread streaming weight columns) and the two epilogues, which the bf16
// MFMA partial kernels share:
//  up-projection (w_up_t [d_ff][d_model], K-contiguous): bias, ReLU,
//    rounding, and the TwELL pack of each (row, tile) under the same rules as
//    the MFMA path ("Sparser, Faster, Lighter Transformer Language Models
//    (Sakana AI + NVIDIA)", Figure 1 description);
//  dense fallback (w_down [d_ff][d_model], N-contiguous): rounding and the
//    scatter to y[dense_rows[m]].
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace twell {
namespace {

constexpr int kSkThreads = 256;
constexpr int kSkKC = 256;      // K per LDS chunk of A, up-projection
constexpr int kSkKCDown = 64;   // K per LDS chunk of A, fallback
constexpr int kSkLoads = 16;    // weight loads a thread keeps in flight
// Partial-sum loads in flight per output: the smallest of 8, 16 and 32 that
// covers the slice count, so the slices are read in one batch (decode layer,
// 24 slices: three batches of 8 one after the other before).
// Granules of the fp32 K split: one batch of weight loads per thread (8 x 4
// columns of a [N][K] row, 16 rows of a [K][N] weight), so a small K is cut
// into slices that each take one round of loads instead of several in turn
// (slice ends stay whole batches: a batch never reads past its slice).
constexpr int kSkSliceNK = 4 * (kSkLoads / 2);
constexpr int kSkSliceKN = kSkLoads;

template <typename E>
struct Vec16B {  // elements of E in 16 bytes
  static constexpr int N = 16 / static_cast<int>(sizeof(E));
};

// N elements of E kept as raw bits (N * sizeof(E) bytes, one vector load),
// converted to float only where they are used.
template <typename E, int N>
struct Raw {
  static constexpr int W = (N * static_cast<int>(sizeof(E)) + 3) / 4;  // 32-bit words
  uint32_t d[W];
  __device__ __forceinline__ void load(const E* p) {
    if constexpr (W == 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(p);
      d[0] = q.x, d[1] = q.y, d[2] = q.z, d[3] = q.w;
    } else if constexpr (W == 2) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      d[0] = q.x, d[1] = q.y;
    } else if constexpr (W == 1 && sizeof(E) * N == 4) {
      d[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) d[w] = reinterpret_cast<const uint32_t*>(p)[w];
    }
  }
  __device__ __forceinline__ float operator[](int i) const {
    if constexpr (sizeof(E) == 2)
      return __uint_as_float((i & 1) ? (d[i >> 1] & 0xffff0000u) : (d[i >> 1] << 16));
    else
      return __uint_as_float(d[i]);
  }
};

// Rows per workgroup of the fp32 partial kernels (R): blockIdx.z picks the
// group of R rows [z * R, ...) of A.  16 as a rule; 4 when the grid would
// otherwise have too few workgroups to spread over the CUs (tiny layers).
constexpr int kSkRows = 16;
constexpr int kSkRowsSmall = 4;
constexpr int kSkMinBlocks = 64;

// Rows [r0, r0 + R) ∩ [0, M) of A[:, k0 .. k0 + KC) into LDS as float
// [R][KC]; other rows and columns >= K are zero.
template <typename E, int KC, int R>
__device__ __forceinline__ void stage_a(float* sA, const E* __restrict__ A, int64_t lda, int r0,
                                        int M, int k0, int K) {
  for (int e = threadIdx.x; e < R * KC; e += kSkThreads) {
    const int m = e / KC, k = e - m * KC;
    float v = 0.f;
    if (r0 + m < M && k0 + k < K)
      v = ElemTraits<E>::to_f32(A[static_cast<int64_t>(r0 + m) * lda + k0 + k]);
    sA[e] = v;
  }
}

// Columns per thread of skinny_kn_partial: 16 bytes of E per weight row.
template <typename E>
constexpr int kn_cols() {
  return 16 / static_cast<int>(sizeof(E));
}

// Weight [K][N] (N-contiguous): thread t owns CPT consecutive columns and
// walks the slice's K range kSkLoads rows at a time, all of a batch's loads
// issued before any is used; the A rows are restaged in LDS every KC.
template <typename E, int R>
__global__ __launch_bounds__(kSkThreads) void skinny_kn_partial(
    const E* __restrict__ A, int64_t lda, const int32_t* __restrict__ m_dev, int m_cap, int K,
    int N, int kw, int mm, const E* __restrict__ W, float* __restrict__ part) {
  constexpr int CPT = kn_cols<E>();
  constexpr int KC = kSkKCDown, U = kSkLoads;
  static_assert(KC % U == 0, "whole load batches per chunk");
  __shared__ __attribute__((aligned(16))) float sA[R * KC];
  const int M = m_dev != nullptr ? min(*m_dev, m_cap) : m_cap;
  const int r0 = blockIdx.z * R;
  if (r0 >= M) return;
  const int slice = blockIdx.y, kbeg = slice * kw, kfin = min(kbeg + kw, K);
  const int n = (blockIdx.x * kSkThreads + threadIdx.x) * CPT;
  const bool live = n < N;  // N is a multiple of 8: a thread's columns are all in or all out
  const int nc = live ? n : 0;
  float acc[R][CPT];
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[m][c] = 0.f;
  for (int k0 = kbeg; k0 < kfin; k0 += KC) {
    __syncthreads();  // the previous chunk's A is no longer read
    stage_a<E, KC, R>(sA, A, lda, r0, M, k0, K);
    __syncthreads();
    const int kend = min(KC, kfin - k0);
    for (int k = 0; k < kend; k += U) {
      Raw<E, CPT> w[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        // rows past the chunk reuse its first row (in bounds); their A values are 0
        const int kr = k + j < kend ? k + j : 0;
        w[j].load(W + static_cast<int64_t>(k0 + kr) * N + nc);
      }
#pragma unroll
      for (int m = 0; m < R; ++m) {
#pragma unroll
        for (int j4 = 0; j4 < U; j4 += 4) {
          const float4 a = *reinterpret_cast<const float4*>(sA + m * KC + k + j4);
          const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[m][c] = fmaf(av[j], w[j4 + j][c], acc[m][c]);
        }
      }
    }
  }
  if (!live) return;
  float* dst = part + (static_cast<int64_t>(slice) * mm + r0) * N + n;
#pragma unroll
  for (int m = 0; m < R; ++m)
    if (r0 + m < M)
#pragma unroll
      for (int c = 0; c < CPT; ++c) dst[static_cast<int64_t>(m) * N + c] = acc[m][c];
}

// Weight [N][K] (K-contiguous): thread t owns column n = one weight row and
// reads the slice's K range 16 bytes at a time, kSkLoads / 2 loads in flight.
template <typename E, int R>
__global__ __launch_bounds__(kSkThreads) void skinny_nk_partial(
    const E* __restrict__ A, int64_t lda, int M, int K, int N, int kw, int mm,
    const E* __restrict__ W, float* __restrict__ part) {
  constexpr int V = Vec16B<E>::N, KC = kSkKC, U = kSkLoads / 2;
  static_assert(KC % (V * U) == 0, "whole load batches per chunk");
  __shared__ __attribute__((aligned(16))) float sA[R * KC];
  const int r0 = blockIdx.z * R;
  const int slice = blockIdx.y, kbeg = slice * kw, kfin = min(kbeg + kw, K);
  const int n = blockIdx.x * kSkThreads + threadIdx.x;
  const bool live = n < N;
  float acc[R];
#pragma unroll
  for (int m = 0; m < R; ++m) acc[m] = 0.f;
  const E* wrow = W + static_cast<int64_t>(live ? n : 0) * K;
  for (int k0 = kbeg; k0 < kfin; k0 += KC) {
    __syncthreads();
    stage_a<E, KC, R>(sA, A, lda, r0, M, k0, K);
    __syncthreads();
    const int kend = min(KC, kfin - k0);  // a multiple of V: K is
    for (int k = 0; k < kend; k += V * U) {
      Raw<E, V> w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // chunks past the slice reread its first chunk (in bounds); their A
        // values in LDS are 0, so they add nothing
        const int kk = k + u * V < kend ? k + u * V : 0;
        w[u].load(wrow + k0 + kk);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
#pragma unroll
          for (int q = 0; q < V; q += 4) {
            const float4 a = *reinterpret_cast<const float4*>(sA + m * KC + k + u * V + q);
            acc[m] = fmaf(a.x, w[u][q], acc[m]);
            acc[m] = fmaf(a.y, w[u][q + 1], acc[m]);
            acc[m] = fmaf(a.z, w[u][q + 2], acc[m]);
            acc[m] = fmaf(a.w, w[u][q + 3], acc[m]);
          }
        }
      }
    }
  }
  if (!live) return;
  float* dst = part + (static_cast<int64_t>(slice) * mm + r0) * N + n;
#pragma unroll
  for (int m = 0; m < R; ++m)
    if (r0 + m < M) dst[static_cast<int64_t>(m) * N] = acc[m];
}

// Sum over the ks <= B slices of part[slice][m][n] (slice stride `stride`),
// in slice order, with all B loads issued before the first add (loads past
// the last slice reread it and are dropped).
template <int B>
__device__ __forceinline__ float slice_sum(const float* __restrict__ p, int ks, int64_t stride) {
  float v[B];
#pragma unroll
  for (int u = 0; u < B; ++u) v[u] = p[static_cast<int64_t>(min(u, ks - 1)) * stride];
  // a scheduling boundary: without it the adds are moved up between the
  // loads and only 8 loads stay in flight
  asm volatile("" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < B; ++u)
    if (u < ks) s += v[u];
  return s;
}

// Fallback epilogue: y[dense_rows[m]][n] = sum over slices, rounded.
template <typename E, int B>
__global__ __launch_bounds__(kSkThreads) void skinny_fallback_reduce(
    const float* __restrict__ part, int ks, int mm, const int32_t* __restrict__ n_dense,
    int m_cap, const int32_t* __restrict__ dense_rows, int64_t y_rows, int N, E* __restrict__ y) {
  const int M = min(*n_dense, m_cap);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kSkThreads + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * N) return;
  const int m = static_cast<int>(i / N), n = static_cast<int>(i - static_cast<int64_t>(m) * N);
  const float s =
      slice_sum<B>(part + static_cast<int64_t>(m) * N + n, ks, static_cast<int64_t>(mm) * N);
  const int64_t r = dense_rows[m];
  if (r >= 0 && r < y_rows) y[r * N + n] = ElemTraits<E>::from_f32(s);
}

// Up-projection epilogue, one workgroup per (tile t, group of 4 rows):
// h[m][t*T + c] = ReLU(sum over slices + b) rounded, staged in LDS, then wave
// w packs row 4 blockIdx.y + w of the tile.
constexpr int kPackRows = kSkThreads / kWave;

template <typename E, int B>
__global__ __launch_bounds__(kSkThreads) void skinny_up_pack(
    const float* __restrict__ part, int ks, int mm, int M, int dff, int T, int C, int nt,
    const float* __restrict__ bias, E* __restrict__ vals, uint8_t* __restrict__ idx,
    uint8_t* __restrict__ cnt, uint8_t* __restrict__ flags, E* __restrict__ spill,
    E* __restrict__ hdebug) {
  constexpr int EPT = kPackRows * 256 / kSkThreads;  // elements per thread, T <= 256
  __shared__ __attribute__((aligned(16))) E sh[kPackRows * 256];
  const int t = blockIdx.x, r0 = blockIdx.y * kPackRows;
  const int rows = min(kPackRows, M - r0);
  const int c0 = t * T;
  const int64_t stride = static_cast<int64_t>(mm) * dff;
  // all slice loads of all of this thread's elements in flight together
  // (the launcher picks B >= ks)
  float z[EPT];
  int64_t off[EPT];
  bool ok[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = threadIdx.x + j * kSkThreads;
    const int m = e / T, c = e - m * T;
    ok[j] = m < rows;
    off[j] = static_cast<int64_t>(ok[j] ? r0 + m : r0) * dff + c0 + (ok[j] ? c : 0);
    z[j] = 0.f;
  }
  {  // ks <= B: one batch; loads past the last slice reread it and are dropped
    float v[EPT][B];
#pragma unroll
    for (int j = 0; j < EPT; ++j)
#pragma unroll
      for (int u = 0; u < B; ++u) v[j][u] = part[min(u, ks - 1) * stride + off[j]];
    asm volatile("" ::: "memory");  // every load issued before the first add
#pragma unroll
    for (int j = 0; j < EPT; ++j)
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (u < ks) z[j] += v[j][u];
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = threadIdx.x + j * kSkThreads;
    if (!ok[j]) continue;
    const int m = e / T, c = e - m * T;
    const float zz = z[j] + bias[c0 + c];
    const E h = ElemTraits<E>::from_f32(zz > 0.f ? zz : 0.f);
    sh[m * T + c] = h;
    if (hdebug != nullptr) hdebug[static_cast<int64_t>(r0 + m) * dff + c0 + c] = h;
  }
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  if (wave < rows) {
    const int m = r0 + wave;
    const int64_t q = static_cast<int64_t>(m) * nt + t;
    pack_tile_from<E>(sh + wave * T, T, C, vals + q * C, idx + q * C, cnt + q, flags + q,
                      spill != nullptr ? spill + static_cast<int64_t>(m) * dff + c0 : nullptr);
  }
}

int rows_bucket(int64_t m) { return m <= 16 ? 16 : m <= 32 ? 32 : 64; }

template <int R>
hipError_t up_f32_rows(const Geometry& g, const float* x, const float* w_up_t, const float* b_up,
                       const PackOut& out, float* part, hipStream_t s) {
  const int M = static_cast<int>(g.n_rows), N = g.d_ff, K = g.d_model;
  const int nb = (N + kSkThreads - 1) / kSkThreads, nz = (M + R - 1) / R;
  const SkinnySplit sp = skinny_split(g.n_rows, K, nb * nz, kSkSliceNK, 512);
  skinny_nk_partial<float, R><<<dim3(nb, sp.slices, nz), kSkThreads, 0, s>>>(
      x, K, M, K, N, sp.kw, sp.mm, w_up_t, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_skinny_up_epilogue<float>(g, sp, part, b_up, out, s);
}

hipError_t up_f32(const Geometry& g, const float* x, const float* w_up_t, const float* b_up,
                  const PackOut& out, float* part, hipStream_t s) {
  const int nb = (g.d_ff + kSkThreads - 1) / kSkThreads;
  const int nz = static_cast<int>((g.n_rows + kSkRows - 1) / kSkRows);
  const SkinnySplit sp = skinny_split(g.n_rows, g.d_model, nb * nz, kSkSliceNK, 512);
  return nb * nz * sp.slices < kSkMinBlocks
             ? up_f32_rows<kSkRowsSmall>(g, x, w_up_t, b_up, out, part, s)
             : up_f32_rows<kSkRows>(g, x, w_up_t, b_up, out, part, s);
}

template <int R>
hipError_t fallback_f32_rows(const Geometry& g, const float* a, const int32_t* dense_rows,
                             const int32_t* n_dense, int m_cap, const float* w_down, float* y,
                             float* part, hipStream_t s) {
  constexpr int CPT = kn_cols<float>();
  const int N = g.d_model, K = g.d_ff;
  const int nb = (N + kSkThreads * CPT - 1) / (kSkThreads * CPT);
  const int nz = (m_cap + R - 1) / R;
  const SkinnySplit sp = skinny_split(g.n_rows, K, nb * nz, kSkSliceKN, 512);
  skinny_kn_partial<float, R><<<dim3(nb, sp.slices, nz), kSkThreads, 0, s>>>(
      a, K, n_dense, m_cap, K, N, sp.kw, sp.mm, w_down, part);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_skinny_fallback_reduce<float>(g, sp, part, n_dense, m_cap, dense_rows, y, s);
}

hipError_t fallback_f32(const Geometry& g, const float* a, const int32_t* dense_rows,
                        const int32_t* n_dense, int m_cap, const float* w_down, float* y,
                        float* part, hipStream_t s) {
  constexpr int CPT = kn_cols<float>();
  const int nb = (g.d_model + kSkThreads * CPT - 1) / (kSkThreads * CPT);
  const int nz = (m_cap + kSkRows - 1) / kSkRows;
  const SkinnySplit sp = skinny_split(g.n_rows, g.d_ff, nb * nz, kSkSliceKN, 512);
  return nb * nz * sp.slices < kSkMinBlocks
             ? fallback_f32_rows<kSkRowsSmall>(g, a, dense_rows, n_dense, m_cap, w_down, y, part, s)
             : fallback_f32_rows<kSkRows>(g, a, dense_rows, n_dense, m_cap, w_down, y, part, s);
}

}  // namespace

// Calls f with the partial-sum batch for `slices` slices (at most 32).
template <class F>
void by_sum_batch(int slices, F&& f) {
  static_assert(kSkinnyMaxSlices <= 32, "one batch of 32 covers every slice count");
  if (slices <= 8) f(std::integral_constant<int, 8>{});
  else if (slices <= 16) f(std::integral_constant<int, 16>{});
  else f(std::integral_constant<int, 32>{});
}

SkinnySplit skinny_split(int64_t n_rows, int K, int n_blocks, int granule, int target_blocks) {
  int want = (target_blocks + n_blocks - 1) / n_blocks;
  want = want < 1 ? 1 : want > kSkinnyMaxSlices ? kSkinnyMaxSlices : want;
  const int units = (K + granule - 1) / granule;
  if (want > units) want = units;
  const int kw = ((units + want - 1) / want) * granule;
  return SkinnySplit{(K + kw - 1) / kw, kw, rows_bucket(n_rows)};
}

size_t skinny_ws_bytes(const Geometry& g) {
  if (g.n_rows <= 0 || g.n_rows > kSkinnyMaxRows) return 0;
  const size_t cols = static_cast<size_t>(g.d_ff > g.d_model ? g.d_ff : g.d_model);
  return static_cast<size_t>(kSkinnyMaxSlices) * rows_bucket(g.n_rows) * cols * sizeof(float);
}

template <typename E>
hipError_t launch_skinny_up_epilogue(const Geometry& g, const SkinnySplit& sp, const float* part,
                                     const float* b_up, const PackOut& out, hipStream_t s) {
  if (g.tile > 256) return hipErrorInvalidValue;  // the tile is staged in LDS
  const unsigned groups = static_cast<unsigned>((g.n_rows + kPackRows - 1) / kPackRows);
  auto go = [&](auto b) {
    skinny_up_pack<E, decltype(b)::value><<<dim3(g.n_tiles, groups), kSkThreads, 0, s>>>(
        part, sp.slices, sp.mm, static_cast<int>(g.n_rows), g.d_ff, g.tile, g.capacity,
        g.n_tiles, b_up, static_cast<E*>(out.vals), out.idx, out.cnt, out.flags,
        static_cast<E*>(out.spill), static_cast<E*>(out.h_debug));
  };
  by_sum_batch(sp.slices, go);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_skinny_fallback_reduce(const Geometry& g, const SkinnySplit& sp,
                                         const float* part, const int32_t* n_dense, int m_cap,
                                         const int32_t* dense_rows, E* y, hipStream_t s) {
  const int64_t outs = static_cast<int64_t>(m_cap) * g.d_model;
  auto go = [&](auto b) {
    skinny_fallback_reduce<E, decltype(b)::value>
        <<<static_cast<unsigned>((outs + kSkThreads - 1) / kSkThreads), kSkThreads, 0, s>>>(
            part, sp.slices, sp.mm, n_dense, m_cap, dense_rows, g.n_rows, g.d_model, y);
  };
  by_sum_batch(sp.slices, go);
  return hipGetLastError();
}

hipError_t launch_skinny_up_pack_f32(const Geometry& g, const float* x, const float* w_up_t,
                                     const float* b_up, const PackOut& out, float* part,
                                     hipStream_t s) {
  return up_f32(g, x, w_up_t, b_up, out, part, s);
}

hipError_t launch_skinny_fallback_f32(const Geometry& g, const float* a, const int32_t* dense_rows,
                                      const int32_t* n_dense, int64_t dense_cap,
                                      const float* w_down, float* y, float* part, hipStream_t s) {
  const int64_t worst = dense_cap < g.n_rows ? dense_cap : g.n_rows;
  if (worst <= 0) return hipSuccess;
  return fallback_f32(g, a, dense_rows, n_dense, static_cast<int>(worst), w_down, y, part, s);
}

template hipError_t launch_skinny_up_epilogue<uint16_t>(const Geometry&, const SkinnySplit&,
                                                        const float*, const float*,
                                                        const PackOut&, hipStream_t);
template hipError_t launch_skinny_up_epilogue<float>(const Geometry&, const SkinnySplit&,
                                                     const float*, const float*, const PackOut&,
                                                     hipStream_t);
template hipError_t launch_skinny_fallback_reduce<uint16_t>(const Geometry&, const SkinnySplit&,
                                                            const float*, const int32_t*, int,
                                                            const int32_t*, uint16_t*,
                                                            hipStream_t);
template hipError_t launch_skinny_fallback_reduce<float>(const Geometry&, const SkinnySplit&,
                                                         const float*, const int32_t*, int,
                                                         const int32_t*, float*, hipStream_t);

}  // namespace twell
