// G3 twell_spmm, sparse part: y[n, :] = sum over the stored slots (t, k) of row
// n of values[n,t,k] * w_down[t*T + indices[n,t,k], :], float32 accumulation.
//
// Only the w_down rows named by stored indices are read, which is how the
// method turns activation sparsity into skipped work ("The Relentless Search
// for Efficiency in Large-Scale Language Models", section "Mechanism of
// Action: Kernel-Level Optimization": kernels that process only the non-zero
// elements; TwELL layout per "Sparser, Faster, Lighter Transformer Language
// Models (Sakana AI + NVIDIA)", Figure 1 description).
//
// One wave per (row, 64-lane column chunk).  The wave reads the row's slots
// 64 at a time (coalesced), ballots the live ones, and walks them with
// readlane so the row index and value are wave-uniform scalars; each live
// slot then costs one coalesced 16-byte load of w_down per lane.
#include "common.h"
#include "kernels.h"

namespace twell {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

template <typename E>
struct SpmmVec;
template <>
struct SpmmVec<uint16_t> {
  static constexpr int N = 8;
};
template <>
struct SpmmVec<float> {
  static constexpr int N = 4;
};

template <typename E>
__device__ __forceinline__ void fma_row(float (&acc)[SpmmVec<E>::N], float v, const uint4& w);

template <>
__device__ __forceinline__ void fma_row<uint16_t>(float (&acc)[8], float v, const uint4& w) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(v, __uint_as_float(d[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(v, __uint_as_float(d[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

template <>
__device__ __forceinline__ void fma_row<float>(float (&acc)[4], float v, const uint4& w) {
  acc[0] = fmaf(v, __uint_as_float(w.x), acc[0]);
  acc[1] = fmaf(v, __uint_as_float(w.y), acc[1]);
  acc[2] = fmaf(v, __uint_as_float(w.z), acc[2]);
  acc[3] = fmaf(v, __uint_as_float(w.w), acc[3]);
}

template <typename E>
__device__ __forceinline__ uint4 store_form(const float (&acc)[SpmmVec<E>::N]);

template <>
__device__ __forceinline__ uint4 store_form<uint16_t>(const float (&acc)[8]) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d[i] = static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * i])) |
           (static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * i + 1])) << 16);
  return make_uint4(d[0], d[1], d[2], d[3]);
}

template <>
__device__ __forceinline__ uint4 store_form<float>(const float (&acc)[4]) {
  return make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                    __float_as_uint(acc[3]));
}

template <typename E>
__global__ __launch_bounds__(kThreads) void spmm_sparse_kernel(
    const E* __restrict__ vals, const uint8_t* __restrict__ idx, const uint8_t* __restrict__ cnt,
    const int32_t* __restrict__ row_map, const E* __restrict__ w, E* __restrict__ y, int64_t N,
    int dm, int T, int C, int nt, int n_chunks) {
  constexpr int V = SpmmVec<E>::N;
  typedef ElemTraits<E> Tr;
  const int lane = lane_id();
  const int64_t items = N * n_chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nslots = nt * C;
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
       item < items; item += stride) {
    const int chunk = static_cast<int>(item / N);
    const int64_t n = item % N;
    if (row_map != nullptr && row_map[n] >= 0) continue;  // dense row: the fallback GEMM writes it
    const int col = chunk * (kWave * V) + lane * V;
    const bool live_col = col < dm;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const int64_t s0 = n * nslots;
    for (int g = 0; g < nslots; g += kWave) {
      const int s = g + lane;
      int j = 0;
      float v = 0.f;
      bool live = false;
      if (s < nslots) {
        const int t = s / C;
        const int k = s - t * C;
        if (k < static_cast<int>(cnt[n * nt + t])) {
          const int local = static_cast<int>(idx[s0 + s]);
          live = local < T;  // a malformed index is ignored rather than read out of bounds
          j = t * T + local;
          v = Tr::to_f32(vals[s0 + s]);
        }
      }
      uint64_t mask = wave_ballot(live);
      while (mask != 0) {
        // up to four live slots per round: four independent loads in flight
        int src[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (mask != 0) {
            src[u] = __builtin_ctzll(mask);
            mask &= mask - 1;
          } else {
            src[u] = -1;
          }
        }
        uint4 wv[4];
        float sv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (src[u] >= 0) {
            const int ju = __builtin_amdgcn_readlane(j, src[u]);
            sv[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src[u]));
            wv[u] = live_col ? *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(ju) * dm + col)
                             : make_uint4(0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (src[u] >= 0) fma_row<E>(acc, sv[u], wv[u]);
      }
    }
    if (live_col) *reinterpret_cast<uint4*>(y + n * dm + col) = store_form<E>(acc);
  }
}

}  // namespace

hipError_t launch_spmm_sparse(const Geometry& g, int elem_bytes, const void* vals,
                              const uint8_t* idx, const uint8_t* cnt, const int32_t* row_map,
                              const void* w_down, void* y, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const int V = elem_bytes == 2 ? 8 : 4;
  const int n_chunks = (g.d_model + kWave * V - 1) / (kWave * V);
  const int64_t items = g.n_rows * n_chunks;
  const int64_t want = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned blocks = static_cast<unsigned>(want < 16384 ? want : 16384);
  if (elem_bytes == 2) {
    spmm_sparse_kernel<uint16_t><<<blocks, kThreads, 0, s>>>(
        static_cast<const uint16_t*>(vals), idx, cnt, row_map, static_cast<const uint16_t*>(w_down),
        static_cast<uint16_t*>(y), g.n_rows, g.d_model, g.tile, g.capacity, g.n_tiles, n_chunks);
  } else {
    spmm_sparse_kernel<float><<<blocks, kThreads, 0, s>>>(
        static_cast<const float*>(vals), idx, cnt, row_map, static_cast<const float*>(w_down),
        static_cast<float*>(y), g.n_rows, g.d_model, g.tile, g.capacity, g.n_tiles, n_chunks);
  }
  return hipGetLastError();
}

}  // namespace twell
