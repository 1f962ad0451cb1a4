// ELLPACK rows (Figure 1(a)) beside TwELL: each token row keeps its non-zeros
// in ascending column order, padded to a fixed width W, with their 16-bit
// column numbers and a per-row count.  It is TwELL with a single tile that
// spans the whole row ("Sparser, Faster, Lighter Transformer Language Models
// (Sakana AI + NVIDIA)", Figure 1 description: panel a is ELL, panel b TwELL,
// panel c the hybrid).  Rows with more than W non-zeros go to the dense
// matrix, as rows with an overflowing tile do in the hybrid TwELL ("Nvidia and
// Sakana make LLMs 30% faster by doing less math", section "Reshaping math for
// the GPU").  A row's slot positions depend on every column of the row, so
// ELL needs a whole-row pass over a materialised h; the tiled up-projection
// cannot emit it from its epilogue the way it emits TwELL.
//
//  ell_count  one wave per row: non-zeros, and the row's overflow flag;
//  (routing)  the TwELL scan with one flag per row numbers the dense rows;
//  ell_fill   one wave per row: a sparse row's non-zeros to its slots in
//             column order (ballot prefix), padding after them; a dense
//             row's full copy to dense_values and all-padding slots;
//  ell_unpack one workgroup per row, the row rebuilt in LDS;
//  ell_spmm   the sparse rows' product from their slot lists (no per-tile
//             compaction: the list is already compact), then the dense
//             fallback GEMM for the dense rows.
#include <type_traits>

#include "../../include/twell.h"
#include "common.h"
#include "kernels.h"
#include "spmm_split.h"

namespace twell {
namespace {

constexpr int kEllThreads = 256;
constexpr int kEllWaves = kEllThreads / kWave;

template <typename E>
struct EllVec {
  static constexpr int N = 16 / sizeof(E);  // elements per 16-byte load
};

// Non-zero count of each row; flag = count > W.  One wave per row, 16-byte
// loads (d_ff is a multiple of 8, so every load is a whole vector).
template <typename E>
__global__ __launch_bounds__(kEllThreads) void ell_count_kernel(const E* __restrict__ h, int64_t N,
                                                                int dff, int W,
                                                                uint8_t* __restrict__ flags) {
  typedef ElemTraits<E> Tr;
  constexpr int V = EllVec<E>::N;
  const int lane = lane_id();
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kEllWaves + threadIdx.x / kWave;
  if (n >= N) return;
  const E* row = h + n * dff;
  int c = 0;
  for (int col = lane * V; col < dff; col += kWave * V) {
    E v[V];
    *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(row + col);
#pragma unroll
    for (int e = 0; e < V; ++e) c += Tr::abs_bits(v[e]) != 0u;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
  if (lane == 0) flags[n] = static_cast<uint8_t>(c > W ? 1 : 0);
}

// Slots of every row (row_map: dense index, or -1 for a sparse row).
template <typename E>
__global__ __launch_bounds__(kEllThreads) void ell_fill_kernel(
    const E* __restrict__ h, int64_t N, int dff, int W, const int32_t* __restrict__ row_map,
    int64_t cap, E* __restrict__ vals, uint16_t* __restrict__ cols, uint16_t* __restrict__ cnt,
    E* __restrict__ dense_values) {
  typedef ElemTraits<E> Tr;
  constexpr int V = EllVec<E>::N;
  const int lane = lane_id();
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kEllWaves + threadIdx.x / kWave;
  if (n >= N) return;
  const E* row = h + n * dff;
  E* sv = vals + n * W;
  uint16_t* sc = cols + n * W;
  const int m = row_map[n];
  int stored = 0;
  if (m >= 0) {  // dense row: a bit copy, when it fits in the dense matrix
    if (m < cap)
      for (int col = lane * V; col < dff; col += kWave * V)
        *reinterpret_cast<uint4*>(dense_values + static_cast<int64_t>(m) * dff + col) =
            *reinterpret_cast<const uint4*>(row + col);
  } else {
    for (int col0 = 0; col0 < dff; col0 += kWave * V) {
      const int col = col0 + lane * V;
      E v[V];
      // every lane takes part in the ballots; lanes past the row's end hold zeros
      *reinterpret_cast<uint4*>(v) =
          col < dff ? *reinterpret_cast<const uint4*>(row + col) : make_uint4(0, 0, 0, 0);
      int mine = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) mine += Tr::abs_bits(v[e]) != 0u;
      // exclusive prefix of the lanes' counts (at most 8: four bit ballots)
      int before = 0, total = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint64_t msk = wave_ballot((mine >> b) & 1);
        before += popc_below(msk) << b;
        total += popc64(msk) << b;
      }
      int p = stored + before;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (Tr::abs_bits(v[e]) != 0u) {  // never past W: the row was counted sparse
          sv[p] = v[e];
          sc[p] = static_cast<uint16_t>(col + e);
          ++p;
        }
      }
      stored += total;
    }
  }
  for (int s = stored + lane; s < W; s += kWave) {  // padding: +0.0 and column 0
    sv[s] = E(0);
    sc[s] = 0;
  }
  if (lane == 0) cnt[n] = static_cast<uint16_t>(stored);
}

// ell_to_dense: one workgroup per row, the row built in LDS (zeros, then the
// slots or the stored dense row) and written out with 16-byte stores.
template <typename E>
__global__ __launch_bounds__(kEllThreads) void ell_unpack_kernel(
    const E* __restrict__ vals, const uint16_t* __restrict__ cols, const uint16_t* __restrict__ cnt,
    const int32_t* __restrict__ dense_rows, const E* __restrict__ dense_values,
    const int32_t* __restrict__ n_dense, int64_t cap, int64_t N, int dff, int W,
    E* __restrict__ h) {
  extern __shared__ uint4 ell_row[];
  constexpr int V = EllVec<E>::N;
  E* buf = reinterpret_cast<E*>(ell_row);
  const int64_t n = blockIdx.x;
  // the stored dense rows are ascending: binary search
  const int64_t stored = min(static_cast<int64_t>(max(*n_dense, 0)), cap);
  int64_t lo = 0, hi = stored;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(dense_rows[mid]) < n) lo = mid + 1;
    else hi = mid;
  }
  E* out = h + n * dff;
  if (lo < stored && dense_rows[lo] == n) {
    for (int col = threadIdx.x * V; col < dff; col += kEllThreads * V)
      *reinterpret_cast<uint4*>(out + col) =
          *reinterpret_cast<const uint4*>(dense_values + lo * dff + col);
    return;
  }
  for (int col = threadIdx.x * V; col < dff; col += kEllThreads * V)
    *reinterpret_cast<uint4*>(buf + col) = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const int c = min(static_cast<int>(cnt[n]), W);
  for (int s = threadIdx.x; s < c; s += kEllThreads) {
    const int col = cols[n * W + s];
    if (col < dff) buf[col] = vals[n * W + s];  // a malformed column is ignored
  }
  __syncthreads();
  for (int col = threadIdx.x * V; col < dff; col += kEllThreads * V)
    *reinterpret_cast<uint4*>(out + col) = *reinterpret_cast<const uint4*>(buf + col);
}

// ---- sparse product of the ELL rows
// bf16, d_model a multiple of 512: the XCD-sliced form of the TwELL kernel
// (each XCD owns a column slice of w_down and y), but a wave copies the row's
// slot list straight into LDS (byte offset of the w_down row, value), since
// an ELL row's live slots are already the first cnt ones.
template <int VEC>
__global__ __launch_bounds__(kEllThreads) void ell_spmm_list_bf16_kernel(
    const uint16_t* __restrict__ vals, const uint16_t* __restrict__ cols,
    const uint16_t* __restrict__ cnt, DenseSkip skip, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ y, int64_t N, int dm, int dff, int W, int n_slices) {
  extern __shared__ uint2 ell_lists[];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  uint2* list = ell_lists + wave * W;
  const int xcd = blockIdx.x % 8;
  const int slice = xcd % n_slices;
  const int parts = 8 / n_slices;  // XCDs sharing this slice split its rows
  const int part = xcd / n_slices;
  const int64_t per_xcd_waves = static_cast<int64_t>(gridDim.x / 8) * kEllWaves;
  const int64_t wid = static_cast<int64_t>(blockIdx.x / 8) * kEllWaves + wave;
  const int col = slice * (kWave * VEC) + lane * VEC;
  const char* wbase = reinterpret_cast<const char*>(w + col);
  for (int64_t n = part + parts * wid; n < N; n += parts * per_xcd_waves) {
    if (listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
    const int nnz = min(static_cast<int>(cnt[n]), W);
    for (int s = lane; s < nnz; s += kWave) {
      const uint32_t c = min(static_cast<uint32_t>(cols[n * W + s]), static_cast<uint32_t>(dff - 1));
      list[s] = make_uint2(c * static_cast<uint32_t>(dm) * 2u, vals[n * W + s]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's list is in LDS
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int k = 0; k < nnz; k += kListUnroll) {
      uint2 e[kListUnroll];
      WVec<VEC> wv[kListUnroll];
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u) {
        e[u] = list[min(k + u, nnz - 1)];  // past the end: reread the last entry, unused
        load_wvec<VEC>(wv[u], reinterpret_cast<const uint16_t*>(wbase + e[u].x));
      }
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u)
        if (k + u < nnz) dot2_row<VEC>(acc, e[u].y, e[u].y << 16, wv[u]);
    }
    uint32_t out[VEC / 2];
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i)
      out[i] = static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * i])) |
               (static_cast<uint32_t>(ElemTraits<uint16_t>::from_f32(acc[2 * i + 1])) << 16);
    uint16_t* dst = y + n * dm + col;
#pragma unroll
    for (int q = 0; q < VEC / 8; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) =
          make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the list is rewritten by the next row after these reads
  }
}

// Any width or dtype: one wave per (row, 64-lane chunk of 16-byte column
// groups); the wave reads 64 slots at a time and walks the live ones, four
// w_down rows in flight.
template <typename E>
__global__ __launch_bounds__(kEllThreads) void ell_spmm_kernel(
    const E* __restrict__ vals, const uint16_t* __restrict__ cols, const uint16_t* __restrict__ cnt,
    DenseSkip skip, const E* __restrict__ w, E* __restrict__ y, int64_t N, int dm, int dff, int W,
    int n_chunks) {
  constexpr int V = SpmmVec<E>::N;
  typedef ElemTraits<E> Tr;
  const int lane = lane_id();
  const int64_t items = N * n_chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kEllWaves;
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * kEllWaves + threadIdx.x / kWave;
       item < items; item += stride) {
    const int chunk = static_cast<int>(item / N);
    const int64_t n = item % N;
    if (listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
    const int col = chunk * (kWave * V) + lane * V;
    const bool live_col = col < dm;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    const int nnz = min(static_cast<int>(cnt[n]), W);
    for (int g = 0; g < nnz; g += kWave) {
      const int s = g + lane;
      int j = 0;
      float v = 0.f;
      if (s < nnz) {
        j = min(static_cast<int>(cols[n * W + s]), dff - 1);
        v = Tr::to_f32(vals[n * W + s]);
      }
      const int live = min(kWave, nnz - g);
      for (int q = 0; q < live; q += 4) {
        uint4 wv[4];
        float sv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int src = min(q + u, live - 1);  // past the end: reread the last slot, unused
          const int ju = __builtin_amdgcn_readlane(j, src);
          sv[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
          wv[u] = live_col ? *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(ju) * dm + col)
                           : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (q + u < live) fma_row<E>(acc, sv[u], wv[u]);
      }
    }
    if (live_col) {
      E o[V];
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] = Tr::from_f32(acc[i]);
      *reinterpret_cast<uint4*>(y + n * dm + col) = *reinterpret_cast<const uint4*>(o);
    }
  }
}

}  // namespace

hipError_t launch_ell_pack(const Geometry& g, int elem_bytes, const void* h, const RouteBufs& rb,
                           void* vals, uint16_t* cols, uint16_t* cnt, int32_t* dense_rows,
                           void* dense_values, int64_t dense_cap, int32_t* n_dense,
                           int32_t* status, hipStream_t s) {
  const int W = g.capacity;
  const unsigned blocks = static_cast<unsigned>((g.n_rows + kEllWaves - 1) / kEllWaves);
  Geometry g1 = g;
  g1.n_tiles = 1;  // one flag per row
  if (g.n_rows == 0)  // the scan alone: no dense rows, status OK
    return launch_route_scan(g1, rb, dense_rows, dense_cap, n_dense, status, s);
  if (elem_bytes == 2)
    ell_count_kernel<uint16_t><<<blocks, kEllThreads, 0, s>>>(static_cast<const uint16_t*>(h),
                                                              g.n_rows, g.d_ff, W, rb.flags);
  else
    ell_count_kernel<float><<<blocks, kEllThreads, 0, s>>>(static_cast<const float*>(h), g.n_rows,
                                                           g.d_ff, W, rb.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_route_scan(g1, rb, dense_rows, dense_cap, n_dense, status, s);
  if (e != hipSuccess) return e;
  if (elem_bytes == 2)
    ell_fill_kernel<uint16_t><<<blocks, kEllThreads, 0, s>>>(
        static_cast<const uint16_t*>(h), g.n_rows, g.d_ff, W, rb.row_map, dense_cap,
        static_cast<uint16_t*>(vals), cols, cnt, static_cast<uint16_t*>(dense_values));
  else
    ell_fill_kernel<float><<<blocks, kEllThreads, 0, s>>>(
        static_cast<const float*>(h), g.n_rows, g.d_ff, W, rb.row_map, dense_cap,
        static_cast<float*>(vals), cols, cnt, static_cast<float*>(dense_values));
  return hipGetLastError();
}

size_t ell_unpack_lds_bytes(const Geometry& g, int elem_bytes) {
  return static_cast<size_t>(g.d_ff) * elem_bytes;
}

hipError_t launch_ell_unpack(const Geometry& g, int elem_bytes, const void* vals,
                             const uint16_t* cols, const uint16_t* cnt, const int32_t* dense_rows,
                             const void* dense_values, const int32_t* n_dense, int64_t dense_cap,
                             void* h, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(g.n_rows);
  const size_t lds = ell_unpack_lds_bytes(g, elem_bytes);
  if (elem_bytes == 2)
    ell_unpack_kernel<uint16_t><<<blocks, kEllThreads, lds, s>>>(
        static_cast<const uint16_t*>(vals), cols, cnt, dense_rows,
        static_cast<const uint16_t*>(dense_values), n_dense, dense_cap, g.n_rows, g.d_ff,
        g.capacity, static_cast<uint16_t*>(h));
  else
    ell_unpack_kernel<float><<<blocks, kEllThreads, lds, s>>>(
        static_cast<const float*>(vals), cols, cnt, dense_rows,
        static_cast<const float*>(dense_values), n_dense, dense_cap, g.n_rows, g.d_ff,
        g.capacity, static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_ell_spmm_sparse(const Geometry& g, int elem_bytes, const void* vals,
                                  const uint16_t* cols, const uint16_t* cnt, const DenseSkip& skip,
                                  const void* w_down, void* y, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const int W = g.capacity;
  if (elem_bytes == 2 && g.d_model % 512 == 0) {
    const int ns = g.d_model / 512;
    int n_slices = 0, vec = 0;
    if (ns == 1 || ns == 2 || ns == 4 || ns == 8) n_slices = ns, vec = 8;
    else if (ns == 16) n_slices = 8, vec = 16;
    const size_t lds = static_cast<size_t>(kEllWaves) * W * 8;
    const bool offsets_fit = static_cast<int64_t>(g.d_ff) * g.d_model * 2 < (int64_t{1} << 32);
    if (n_slices > 0 && lds <= 64 * 1024 && offsets_fit) {
      const int64_t rows_per_xcd = (g.n_rows + (8 / n_slices) - 1) / (8 / n_slices);
      const int64_t wg_per_xcd = (rows_per_xcd + kEllWaves - 1) / kEllWaves;
      const unsigned blocks = static_cast<unsigned>(8 * (wg_per_xcd < 512 ? wg_per_xcd : 512));
      const uint16_t* v16 = static_cast<const uint16_t*>(vals);
      if (vec == 8)
        ell_spmm_list_bf16_kernel<8><<<blocks, kEllThreads, lds, s>>>(
            v16, cols, cnt, skip, static_cast<const uint16_t*>(w_down),
            static_cast<uint16_t*>(y), g.n_rows, g.d_model, g.d_ff, W, n_slices);
      else
        ell_spmm_list_bf16_kernel<16><<<blocks, kEllThreads, lds, s>>>(
            v16, cols, cnt, skip, static_cast<const uint16_t*>(w_down),
            static_cast<uint16_t*>(y), g.n_rows, g.d_model, g.d_ff, W, n_slices);
      return hipGetLastError();
    }
  }
  const int V = elem_bytes == 2 ? SpmmVec<uint16_t>::N : SpmmVec<float>::N;
  const int n_chunks = (g.d_model + kWave * V - 1) / (kWave * V);
  const int64_t want = (g.n_rows * n_chunks + kEllWaves - 1) / kEllWaves;
  const unsigned blocks = static_cast<unsigned>(want < 16384 ? want : 16384);
  if (elem_bytes == 2)
    ell_spmm_kernel<uint16_t><<<blocks, kEllThreads, 0, s>>>(
        static_cast<const uint16_t*>(vals), cols, cnt, skip, static_cast<const uint16_t*>(w_down),
        static_cast<uint16_t*>(y), g.n_rows, g.d_model, g.d_ff, W, n_chunks);
  else
    ell_spmm_kernel<float><<<blocks, kEllThreads, 0, s>>>(
        static_cast<const float*>(vals), cols, cnt, skip, static_cast<const float*>(w_down),
        static_cast<float*>(y), g.n_rows, g.d_model, g.d_ff, W, n_chunks);
  return hipGetLastError();
}

}  // namespace twell
