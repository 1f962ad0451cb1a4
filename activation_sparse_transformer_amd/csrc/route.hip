// Row routing and the dense <-> TwELL conversions.
//
//  G2a route_scan   per-row OR of the tile-overflow flags (row_or for more
//                   than 1024 rows), ascending numbering of the dense rows
//                   (one workgroup, block-wide prefix scan, so the order is
//                   deterministic);
//  G2b materialize  dense_values[m] = full row of h for each dense row, then
//                   the row's TwELL slots are cleared;
//  G5  pack_tiles   dense_to_twell of an existing h, one wave per (row, tile);
//  G6  unpack       twell_to_dense.
//
// Format: "Sparser, Faster, Lighter Transformer Language Models (Sakana AI +
// NVIDIA)", Figure 1 description (values, tile-local indices, per-tile
// counts; the hybrid splits rows between TwELL and a dense matrix).  The
// conversions are the dense-to-TwELL and TwELL-to-dense paths named in
// "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse Transformers Run Like
// They Were Built for Hopper", section "TwELL: The Packing Format That Fits
// the Machine".  Rows go dense as a whole when any tile overflows (the rare
// dense tokens of "Nvidia and Sakana make LLMs 30% faster by doing less
// math", section "Reshaping math for the GPU").
#include <type_traits>

#include "../../include/twell.h"
#include "common.h"
#include "kernels.h"
#include "spmm_split.h"

namespace twell {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kRowThreads = 256;
constexpr int64_t kPrefixMaxRows = 16384;
// Workgroups of the listed dense-row build (at most one per row; measured at
// 1853 dense rows of 4096: 2048 and 4096 alike, 1024 0.4 us slower).
constexpr int64_t kListedGrid = 2048;

__device__ __forceinline__ bool row_has_flag(const uint8_t* __restrict__ f, int nt) {
  uint32_t any = 0;
  if ((nt & 15) == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(f);
    for (int i = 0; i < nt / 16; ++i) {
      const uint4 q = p[i];
      any |= q.x | q.y | q.z | q.w;
    }
  } else if ((nt & 3) == 0) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(f);
    for (int i = 0; i < nt / 4; ++i) any |= p[i];
  } else {
    for (int i = 0; i < nt; ++i) any |= f[i];
  }
  return any != 0;
}

// Inclusive scan of one int across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// One thread per row: does any tile of the row overflow?  With `blk_cnt`,
// each workgroup also stores how many of its kRowThreads rows are dense.
__global__ __launch_bounds__(kRowThreads) void row_or_kernel(const uint8_t* __restrict__ flags,
                                                             int64_t N, int nt,
                                                             uint8_t* __restrict__ row_dense,
                                                             int32_t* __restrict__ blk_cnt) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x;
  const bool d = n < N && row_has_flag(flags + n * nt, nt);
  if (n < N) row_dense[n] = d ? 1 : 0;
  if (blk_cnt != nullptr) {
    const int c = __syncthreads_count(d);
    if (threadIdx.x == 0) blk_cnt[blockIdx.x] = c;
  }
}

// One workgroup: thread i takes a run of consecutive rows (with `flags`, it
// first ORs each row's tile flags into row_dense; otherwise row_dense is
// given), then a block-wide prefix scan of the per-thread dense counts
// numbers the dense rows in ascending order.
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(
    const uint8_t* __restrict__ flags, int nt, uint8_t* __restrict__ row_dense, int64_t N,
    int32_t* __restrict__ row_map, int32_t* __restrict__ dense_rows, int64_t cap,
    int32_t* __restrict__ n_dense, int32_t* __restrict__ sparse_rows,
    int32_t* __restrict__ n_sparse, int32_t* __restrict__ status) {
  __shared__ int wave_tot[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t per = (N + kScanThreads - 1) / kScanThreads;
  const int64_t r0 = min(N, tid * per), r1 = min(N, r0 + per);
  int local = 0;
  for (int64_t n = r0; n < r1; ++n) {
    uint8_t d;
    if (flags != nullptr) {
      d = row_has_flag(flags + n * nt, nt) ? 1 : 0;
      row_dense[n] = d;
    } else {
      d = row_dense[n];
    }
    local += d;
  }
  const int incl = wave_inclusive_scan(local);
  const int wave = tid / kWave, lane = lane_id();
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kScanThreads / kWave; ++w) {
    before += (w < wave) ? wave_tot[w] : 0;
    total += wave_tot[w];
  }
  int m = before + incl - local;  // dense rows before this thread's first row
  for (int64_t n = r0; n < r1; ++n) {
    if (row_dense[n]) {
      row_map[n] = m;
      if (m < cap) dense_rows[m] = static_cast<int32_t>(n);
      ++m;
    } else {
      row_map[n] = -1;
      sparse_rows[n - m] = static_cast<int32_t>(n);  // sparse rows before n = n - m
    }
  }
  if (tid == 0) {
    *n_dense = total;
    *n_sparse = static_cast<int32_t>(N - total);
    if (status != nullptr) *status = total > cap ? TWELL_ERR_DENSE_CAPACITY : TWELL_OK;
  }
}

template <typename E>
struct Vec16 {
  static constexpr int N = 16 / sizeof(E);
  E v[N];
};

template <typename E>
__device__ __forceinline__ void load_vec(Vec16<E>& d, const E* p) {
  *reinterpret_cast<uint4*>(d.v) = *reinterpret_cast<const uint4*>(p);
}
template <typename E>
__device__ __forceinline__ void store_vec(E* p, const Vec16<E>& d) {
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(d.v);
}

// Columns [c, c + 16/sizeof(E)) of a TwELL row, rebuilt from the slots of
// tile t: zeros except the stored entries.
template <typename E>
__device__ __forceinline__ void gather_tile_vec(Vec16<E>& out, const E* __restrict__ vals,
                                                const uint8_t* __restrict__ idx, int count, int C,
                                                int local0) {
#pragma unroll
  for (int i = 0; i < Vec16<E>::N; ++i) out.v[i] = E(0);
  for (int k = 0; k < count && k < C; ++k) {
    const int d = static_cast<int>(idx[k]) - local0;
    if (d >= 0 && d < Vec16<E>::N) out.v[d] = vals[k];
  }
}

// Routing of at most 64 rows inside a workgroup of at least 64 threads:
// every workgroup ORs the tile flags of all rows into LDS, and one ballot over
// the rows gives each dense row its index (dense rows below it, so ascending
// token order).  Workgroup 0 also writes the dense-row list, the sparse-row
// list, their counts and the status word, as the scan would.  Returns the
// dense index of row n, or -1 for a sparse row.
__device__ int route_rows_in_block(const RouteOut& ro, const uint8_t* __restrict__ flags, int nt,
                                   int64_t cap, int64_t n) {
  __shared__ uint8_t s_rd[kWave];
  __shared__ uint64_t s_mask;
  const int N = static_cast<int>(ro.n_rows);  // at most 64
  if (threadIdx.x < kWave) s_rd[threadIdx.x] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < N * nt; i += blockDim.x)
    if (flags[i]) s_rd[i / nt] = 1;  // every writer stores 1
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int r = threadIdx.x;
    const bool d = r < N && s_rd[r] != 0;
    const uint64_t mask = wave_ballot(d);
    if (r == 0) s_mask = mask;
    if (n == 0 && r < N) {
      const int below = popc_below(mask);  // dense rows below row r
      if (d) {
        if (below < cap) ro.dense_rows[below] = r;
      } else {
        ro.sparse_rows[r - below] = r;
      }
      if (r == 0) {
        const int total = popc64(mask);
        *ro.n_dense = total;
        *ro.n_sparse = N - total;
        if (ro.status != nullptr) *ro.status = total > cap ? TWELL_ERR_DENSE_CAPACITY : TWELL_OK;
      }
    }
  }
  __syncthreads();
  const uint64_t mask = s_mask;
  return ((mask >> n) & 1u) ? popc64(mask & ((uint64_t{1} << n) - 1u)) : -1;
}

// Routing once row_dense and the per-block dense counts are known
// (row_or_kernel): workgroup n counts the dense rows below row n itself, as
// the counts of the kRowThreads-row blocks below n's block plus the rows of
// its own block below it (row_dense holds 0 or 1 per row, so the popcount of
// each 16-byte piece counts them), writes its own entry of the dense-row or
// the sparse-row list, and the last row's workgroup writes the counts and the
// status word.  Returns the dense index of row n, or -1.
__device__ int route_rows_prefix(const RouteOut& ro, int64_t cap, int64_t n) {
  __shared__ int s_part[1024 / kWave];  // up to 1024 threads
  const uint8_t* rd = ro.row_dense;
  const int64_t b = n / kRowThreads, r0 = b * kRowThreads;
  int c = 0;
  for (int64_t i = threadIdx.x; i < b; i += blockDim.x) c += ro.blk_cnt[i];
  for (int64_t i = r0 + static_cast<int64_t>(threadIdx.x) * 16; i < n;
       i += static_cast<int64_t>(blockDim.x) * 16) {
    if (i + 16 <= n) {
      const uint4 v = *reinterpret_cast<const uint4*>(rd + i);
      c += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
    } else {
      for (int64_t j = i; j < n; ++j) c += rd[j];
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) c += __shfl_xor(c, o, kWave);
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = c;
  __syncthreads();
  int below = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) below += s_part[w];
  const int d = rd[n] != 0;
  if (threadIdx.x == 0) {
    if (d) {
      if (below < cap) ro.dense_rows[below] = static_cast<int32_t>(n);
    } else {
      ro.sparse_rows[n - below] = static_cast<int32_t>(n);
    }
    if (n == ro.n_rows - 1) {
      const int64_t total = static_cast<int64_t>(below) + d;
      *ro.n_dense = static_cast<int32_t>(total);
      *ro.n_sparse = static_cast<int32_t>(ro.n_rows - total);
      if (ro.status != nullptr) *ro.status = total > cap ? TWELL_ERR_DENSE_CAPACITY : TWELL_OK;
    }
  }
  return d ? below : -1;
}

// Dense index of row n: from the scan's row map (RM 0), routed inside the
// workgroup (RM 1, at most 64 rows), or from the count of dense rows below
// (RM 2).
template <int RM>
__device__ __forceinline__ int row_dense_index(const RouteOut& ro, const int32_t* row_map,
                                               const uint8_t* flags, int nt, int64_t cap,
                                               int64_t n) {
  if constexpr (RM == 1) return route_rows_in_block(ro, flags, nt, cap, n);
  else if constexpr (RM == 2) return route_rows_prefix(ro, cap, n);
  else return row_map[n];
}

// Dense row n, the m-th: when m < cap, its dense_values row is written from
// full_src, or rebuilt from the row's slots and spilled tiles (in the LDS row
// buffer `rowbuf` when IN_LDS); then the row's TwELL slots are cleared.
// Every thread of the workgroup takes part; it ends on no barrier.
template <typename E, bool IN_LDS, int NT>
__device__ __forceinline__ void build_dense_row(
    int64_t n, int m, E* rowbuf, int dff, int T, int C, int nt, const uint8_t* __restrict__ flags,
    const E* __restrict__ spill, const E* __restrict__ full_src, E* __restrict__ vals,
    uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt, E* __restrict__ dense_values,
    int64_t cap) {
  constexpr int V = Vec16<E>::N;
  const int64_t slot0 = n * nt;
  const int nslots = nt * C;
  if (m < cap) {
    E* dst = dense_values + static_cast<int64_t>(m) * dff;
    if (full_src != nullptr) {
      for (int c = threadIdx.x * V; c < dff; c += NT * V) {
        Vec16<E> o;
        load_vec(o, full_src + n * dff + c);
        store_vec(dst + c, o);
      }
    } else if (!IN_LDS) {  // row too long for LDS: rebuild each 16 bytes from the tile's slots
      for (int c = threadIdx.x * V; c < dff; c += NT * V) {
        Vec16<E> o;
        const int t = c / T;
        if (flags[slot0 + t]) {
          load_vec(o, spill + n * dff + c);
        } else {
          const int64_t s = (slot0 + t) * C;
          gather_tile_vec(o, vals + s, idx + s, cnt[slot0 + t], C, c - t * T);
        }
        store_vec(dst + c, o);
      }
    } else {
      for (int c = threadIdx.x * V; c < dff; c += NT * V) {
        Vec16<E> z;
#pragma unroll
        for (int i = 0; i < V; ++i) z.v[i] = E(0);
        store_vec(rowbuf + c, z);
      }
      __syncthreads();
      for (int s = threadIdx.x; s < nslots; s += NT) {
        const int t = s / C;
        // count, index and value loaded together: no load waits on another
        const int count = cnt[slot0 + t];
        const int local = idx[slot0 * C + s];
        const E v = vals[slot0 * C + s];
        if (s - t * C < count && local < T) rowbuf[t * T + local] = v;
      }
      __syncthreads();
      for (int c = threadIdx.x * V; c < dff; c += NT * V) {
        // a plain 16-byte value (an array loaded from either address space
        // would be kept in scratch memory)
        const uint4 o = flags[slot0 + c / T] ? *reinterpret_cast<const uint4*>(spill + n * dff + c)
                                             : *reinterpret_cast<const uint4*>(rowbuf + c);
        *reinterpret_cast<uint4*>(dst + c) = o;
      }
    }
  }
  __syncthreads();  // every read of this row's slots is done before they are cleared
  for (int64_t i = threadIdx.x; i < nslots; i += NT) {
    vals[slot0 * C + i] = E(0);
    idx[slot0 * C + i] = 0;
  }
  for (int i = threadIdx.x; i < nt; i += NT) cnt[slot0 + i] = 0;
}

// One workgroup per row.  A dense row is assembled in LDS (zeros, then the
// stored slots scattered in), then written out 16 bytes per thread, taking the
// overflowing tiles from the spill area; with `full_src` the row is copied
// from h as is.  Finally the row's TwELL slots are cleared.
//
// With `sp.w_down` set (float32, rows routed in the workgroup, built in LDS,
// 1024 threads), a sparse row's workgroup computes the row's y instead of
// leaving: its 16 waves take the row's 16 tile ranges, as the separate few-row
// sparse kernel does, so y is the same bits.  sp_dm, sp_tpw, sp_chunks:
// d_model, tiles per range, 64-lane column chunks.
template <typename E, bool IN_LDS, int RM, int NT = kRowThreads>
__global__ __launch_bounds__(NT) void materialize_kernel(
    int dff, int T, int C, int nt, const int32_t* __restrict__ row_map,
    const uint8_t* __restrict__ flags, const E* __restrict__ spill, const E* __restrict__ full_src,
    E* __restrict__ vals, uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
    E* __restrict__ dense_values, int64_t cap, RouteOut ro, BuildSpmm sp, int sp_dm, int sp_tpw,
    int sp_chunks) {
  extern __shared__ __attribute__((aligned(16))) unsigned char mat_lds[];
  E* rowbuf = reinterpret_cast<E*>(mat_lds);
  const int64_t n = blockIdx.x;
  const int m = row_dense_index<RM>(ro, row_map, flags, nt, cap, n);
  if (m < 0) {
    if constexpr (IN_LDS && RM == 1 && NT == kSplitParts * kWave &&
                  std::is_same<E, float>::value) {
      if (sp.w_down != nullptr) {
        uint2* lists = reinterpret_cast<uint2*>(mat_lds);
        float* red = reinterpret_cast<float*>(lists + kSplitParts * sp_tpw * C);
        for (int chunk = 0; chunk < sp_chunks; ++chunk)
          spmm_split_row_chunk<E, kSplitParts, 1>(vals, idx, cnt, n,
                                                  static_cast<const E*>(sp.w_down),
                                                  static_cast<E*>(sp.y), sp_dm, T, C, nt, sp_tpw,
                                                  chunk, lists, red);
      }
    }
    return;
  }
  build_dense_row<E, IN_LDS, NT>(n, m, rowbuf, dff, T, C, nt, flags, spill, full_src, vals, idx,
                                  cnt, dense_values, cap);
}

// Routing and dense-row build once row_dense and the per-block dense counts
// are known (row_or_kernel), with workgroups for the dense rows only:
// * every workgroup adds up the blocks' counts (one wave scan) into the
//   offsets of each kRowThreads-row block's dense rows;
// * workgroup b < (row blocks) writes block b's entries of the dense-row and
//   sparse-row lists (a ballot prefix over the block's row flags), and the
//   last block's workgroup the counts and the status word;
// * workgroup b then builds dense rows b, b + G, ... of the n_dense, finding
//   the m-th dense row from the block offsets and a ballot over that block's
//   row flags.
// The lists and dense_values are the same as the one-workgroup-per-row build
// writes; only workgroups that have a dense row to build or a block to list
// do more than read the counts.
template <typename E, bool IN_LDS>
__global__ __launch_bounds__(kRowThreads) void materialize_listed_kernel(
    int dff, int T, int C, int nt, const uint8_t* __restrict__ flags, const E* __restrict__ spill,
    const E* __restrict__ full_src, E* __restrict__ vals, uint8_t* __restrict__ idx,
    uint8_t* __restrict__ cnt, E* __restrict__ dense_values, int64_t cap, RouteOut ro) {
  static_assert(kRowThreads == 4 * kWave, "four waves per workgroup");
  constexpr int kMaxBlocks = static_cast<int>(kPrefixMaxRows / kRowThreads);
  static_assert(kMaxBlocks <= kWave, "one wave scans the block counts");
  extern __shared__ __attribute__((aligned(16))) unsigned char mat_lds[];
  __shared__ int s_off[kMaxBlocks + 1];
  __shared__ int s_wave[kRowThreads / kWave];
  __shared__ int s_blk;
  __shared__ int64_t s_row;
  const int64_t N = ro.n_rows;
  const int nb = static_cast<int>((N + kRowThreads - 1) / kRowThreads);
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (wave == 0) {
    int c = lane < nb ? ro.blk_cnt[lane] : 0;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(c, o, kWave);
      if (lane >= o) c += u;
    }
    // s_off[b]: the dense rows in blocks 0 .. b-1 (s_off[nb]: all of them)
    if (lane == 0) s_off[0] = 0;
    if (lane < nb) s_off[lane + 1] = c;
  }
  __syncthreads();
  const int n_dense = s_off[nb];
  // the rank of each row's flag among the dense rows of its block below it
  auto block_rank = [&](int64_t r0, bool& d) {
    const int64_t r = r0 + threadIdx.x;
    d = r < N && ro.row_dense[r] != 0;
    const uint64_t bal = wave_ballot(d);
    if (lane == 0) s_wave[wave] = popc64(bal);
    __syncthreads();
    int below = popc_below(bal);
    for (int w = 0; w < wave; ++w) below += s_wave[w];
    return below;
  };
  if (static_cast<int>(blockIdx.x) < nb) {
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowThreads;
    bool d;
    const int m = s_off[blockIdx.x] + block_rank(r0, d);
    const int64_t r = r0 + threadIdx.x;
    if (r < N) {
      if (d) {
        if (m < cap) ro.dense_rows[m] = static_cast<int32_t>(r);
      } else {
        ro.sparse_rows[r - m] = static_cast<int32_t>(r);
      }
    }
    if (static_cast<int>(blockIdx.x) == nb - 1 && threadIdx.x == 0) {
      *ro.n_dense = n_dense;
      *ro.n_sparse = static_cast<int32_t>(N - n_dense);
      if (ro.status != nullptr) *ro.status = n_dense > cap ? TWELL_ERR_DENSE_CAPACITY : TWELL_OK;
    }
    __syncthreads();  // s_wave is reused below
  }
  for (int m = blockIdx.x; m < n_dense; m += gridDim.x) {
    // the block holding the m-th dense row, then the row within it
    if (threadIdx.x == 0) s_row = -1;
    if (threadIdx.x < nb && s_off[threadIdx.x] <= m && m < s_off[threadIdx.x + 1])
      s_blk = threadIdx.x;
    __syncthreads();
    const int b = s_blk;
    bool d;
    const int k = block_rank(static_cast<int64_t>(b) * kRowThreads, d);
    if (d && k == m - s_off[b]) s_row = static_cast<int64_t>(b) * kRowThreads + threadIdx.x;
    __syncthreads();
    if (s_row < 0) break;  // (never: the counts come from the same flags)
    build_dense_row<E, IN_LDS, kRowThreads>(s_row, m, reinterpret_cast<E*>(mat_lds), dff, T, C,
                                            nt, flags, spill, full_src, vals, idx, cnt,
                                            dense_values, cap);
    __syncthreads();  // s_blk, s_row, s_wave and the row buffer are reused
  }
}

// Dense-row build for capacities of 4 or 8 slots: one workgroup per row,
// each thread rebuilding 16-byte pieces of the row directly, four at a time.
// A piece of a spilled tile is copied from the spill area; otherwise it is
// zeros plus the tile's stored entries that fall in it, taken from the whole
// slot group loaded with one vector load each for indices and values.  Then
// the row's slots are cleared.
template <int CC, typename E>
struct SlotGroup {
  uint8_t idx[CC];
  E val[CC];
};

template <int CC, typename E>
__device__ __forceinline__ void load_slots(SlotGroup<CC, E>& g, const uint8_t* __restrict__ idx,
                                           const E* __restrict__ vals) {
  static_assert(CC == 4 || CC == 8, "4 or 8 slots");
  if constexpr (CC == 4)
    *reinterpret_cast<uint32_t*>(g.idx) = *reinterpret_cast<const uint32_t*>(idx);
  else
    *reinterpret_cast<uint2*>(g.idx) = *reinterpret_cast<const uint2*>(idx);
  constexpr int VB = CC * static_cast<int>(sizeof(E));  // 8, 16 or 32 bytes
  if constexpr (VB == 8) {
    *reinterpret_cast<uint2*>(g.val) = *reinterpret_cast<const uint2*>(vals);
  } else {
#pragma unroll
    for (int h = 0; h < VB / 16; ++h)
      reinterpret_cast<uint4*>(g.val)[h] = reinterpret_cast<const uint4*>(vals)[h];
  }
}

// Rows routed as row_dense_index says.
template <typename E, int CC, int NT, int RM>
__global__ __launch_bounds__(NT) void materialize_slots_kernel(
    int dff, int T, int nt, const int32_t* __restrict__ row_map, const uint8_t* __restrict__ flags,
    const E* __restrict__ spill, E* __restrict__ vals, uint8_t* __restrict__ idx,
    uint8_t* __restrict__ cnt, E* __restrict__ dense_values, int64_t cap, RouteOut ro) {
  constexpr int V = Vec16<E>::N, B = 4;
  const int64_t n = blockIdx.x;
  const int m = row_dense_index<RM>(ro, row_map, flags, nt, cap, n);
  if (m < 0) return;
  const int64_t slot0 = n * nt;
  if (m < cap) {
    E* dst = dense_values + static_cast<int64_t>(m) * dff;
    for (int base = threadIdx.x * V; base < dff; base += B * NT * V) {
      int t[B], count[B];
      uint8_t f[B];
      SlotGroup<CC, E> sg[B];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int c = min(base + j * NT * V, dff - V);  // past the end: reread, unused
        t[j] = c / T;
        f[j] = flags[slot0 + t[j]];
        count[j] = cnt[slot0 + t[j]];
        load_slots<CC, E>(sg[j], idx + (slot0 + t[j]) * CC, vals + (slot0 + t[j]) * CC);
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int c = base + j * NT * V;
        if (c >= dff) break;
        Vec16<E> o;
        if (f[j]) {
          load_vec(o, spill + n * dff + c);
        } else {
          const int local0 = c - t[j] * T;
#pragma unroll
          for (int i = 0; i < V; ++i) o.v[i] = E(0);
#pragma unroll
          for (int k = 0; k < CC; ++k) {
            const int d = static_cast<int>(sg[j].idx[k]) - local0;
            if (k < count[j] && d >= 0 && d < V) o.v[d] = sg[j].val[k];
          }
        }
        store_vec(dst + c, o);
      }
    }
  }
  __syncthreads();  // every read of this row's slots is done before they are cleared
  const int nslots = nt * CC;
  for (int i = threadIdx.x; i < nslots; i += NT) {
    vals[slot0 * CC + i] = E(0);
    idx[slot0 * CC + i] = 0;
  }
  for (int i = threadIdx.x; i < nt; i += NT) cnt[slot0 + i] = 0;
}

// One wave per (row, tile) of an existing h, kPackAhead consecutive (row,
// tile) pairs at a time (up to 2 KB of h in one piece): the loads of all of
// them are issued before any is packed.  Measured at 16384 x 28672 (T 256):
// one pair at a time 0.570 ms for the whole pack, four pairs a grid stride
// apart 0.560, four consecutive 0.544, eight consecutive 0.594.
constexpr int kPackAhead = 4;

template <typename E, int EPL>
__global__ __launch_bounds__(kRowThreads) void pack_tiles_kernel(
    const E* __restrict__ h, int64_t pairs, int dff, int T, int C, int nt, E* __restrict__ vals,
    uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt, uint8_t* __restrict__ flags) {
  const int lane = lane_id();
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kRowThreads / kWave);
  const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * (kRowThreads / kWave) + threadIdx.x / kWave;
  for (int64_t q0 = wave_id * kPackAhead; q0 < pairs; q0 += waves * kPackAhead) {
    E v[kPackAhead][EPL];
#pragma unroll
    for (int u = 0; u < kPackAhead; ++u) {
      const int64_t q = min(q0 + u, pairs - 1);  // past the end: reread, not packed
      const int64_t n = q / nt;
      const int t = static_cast<int>(q - n * nt);
      const E* src = h + n * dff + static_cast<int64_t>(t) * T + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[u][e] = src[e];
    }
#pragma unroll
    for (int u = 0; u < kPackAhead; ++u) {
      const int64_t q = q0 + u;
      if (q < pairs)
        pack_tile<E, EPL>(v[u], C, vals + q * C, idx + q * C, cnt + q, flags + q, nullptr);
    }
  }
}

template <typename E>
__global__ __launch_bounds__(kRowThreads) void unpack_kernel(
    int dff, int T, int C, int nt, const E* __restrict__ vals, const uint8_t* __restrict__ idx,
    const uint8_t* __restrict__ cnt, const int32_t* __restrict__ dense_rows,
    const E* __restrict__ dense_values, const int32_t* __restrict__ n_dense, int64_t cap,
    E* __restrict__ h) {
  constexpr int V = Vec16<E>::N;
  __shared__ int found;
  const int64_t n = blockIdx.x;
  if (threadIdx.x == 0) {
    // dense_rows[0 .. stored) is strictly ascending: binary search for n.
    int64_t lo = 0, hi = min(static_cast<int64_t>(*n_dense), cap);
    int res = -1;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      const int64_t r = dense_rows[mid];
      if (r == n) {
        res = static_cast<int>(mid);
        break;
      }
      if (r < n) lo = mid + 1; else hi = mid;
    }
    found = res;
  }
  __syncthreads();
  const int m = found;
  E* dst = h + n * dff;
  if (m >= 0) {
    const E* src = dense_values + static_cast<int64_t>(m) * dff;
    for (int c = threadIdx.x * V; c < dff; c += kRowThreads * V) {
      Vec16<E> o;
      load_vec(o, src + c);
      store_vec(dst + c, o);
    }
    return;
  }
  const int64_t slot0 = n * nt;
  for (int c = threadIdx.x * V; c < dff; c += kRowThreads * V) {
    const int t = c / T;
    const int64_t s = (slot0 + t) * C;
    Vec16<E> o;
    gather_tile_vec(o, vals + s, idx + s, cnt[slot0 + t], C, c - t * T);
    store_vec(dst + c, o);
  }
}

}  // namespace

hipError_t launch_route_scan(const Geometry& g, const RouteBufs& rb, int32_t* dense_rows,
                             int64_t dense_cap, int32_t* n_dense, int32_t* status, hipStream_t s) {
  // Up to one row per scan thread the scan ORs the flags itself; beyond
  // that a row-parallel pass does it first.
  const bool fused = g.n_rows <= kScanThreads;
  if (!fused) {
    const unsigned blocks = static_cast<unsigned>((g.n_rows + kRowThreads - 1) / kRowThreads);
    row_or_kernel<<<blocks, kRowThreads, 0, s>>>(rb.flags, g.n_rows, g.n_tiles, rb.row_dense,
                                                 nullptr);
  }
  route_scan_kernel<<<1, kScanThreads, 0, s>>>(fused ? rb.flags : nullptr, g.n_tiles, rb.row_dense, g.n_rows,
                                               rb.row_map, dense_rows, dense_cap, n_dense,
                                               rb.sparse_rows, rb.n_sparse, status);
  return hipGetLastError();
}

int route_mode(const Geometry& g) {
  if (g.n_rows > 0 && g.n_rows <= kSkinnyMaxRows) return 1;
  // above the scan's fused range the row pass runs anyway; each build
  // workgroup then reads at most kPrefixMaxRows bytes of row flags
  if (g.n_rows > kScanThreads && g.n_rows <= kPrefixMaxRows) return 2;
  return 0;
}

hipError_t launch_route_materialize(const Geometry& g, int elem_bytes, const RouteBufs& rb,
                                    const void* spill, const void* full_src, void* vals,
                                    uint8_t* idx, uint8_t* cnt, int32_t* dense_rows,
                                    void* dense_values, int64_t dense_cap, int32_t* n_dense,
                                    int32_t* status, hipStream_t s, const BuildSpmm* sp) {
  const int mode = route_mode(g);
  if (mode == 0) return hipErrorInvalidValue;
  if (mode == 2) {
    const unsigned blocks = static_cast<unsigned>((g.n_rows + kRowThreads - 1) / kRowThreads);
    // the row map is not used in this mode: its first entries hold the per-block counts
    row_or_kernel<<<blocks, kRowThreads, 0, s>>>(rb.flags, g.n_rows, g.n_tiles, rb.row_dense,
                                                 rb.row_map);
  }
  const RouteOut ro{g.n_rows, dense_rows, n_dense, rb.sparse_rows, rb.n_sparse, status,
                    mode == 2 ? rb.row_dense : nullptr, mode == 2 ? rb.row_map : nullptr};
  return launch_materialize(g, elem_bytes, nullptr, rb.flags, spill, full_src, vals, idx, cnt,
                            dense_values, dense_cap, s, &ro, sp);
}

namespace {
// The few-row sparse product as a float32 dense-row build runs it: 16 waves,
// one tile range each, and the LDS for their slot lists and range sums.
struct BuildSpmmPlan {
  int tpw, n_chunks;
  size_t lds_bytes;
};
BuildSpmmPlan build_spmm_plan(const Geometry& g) {
  constexpr int V = 4;  // float32 columns per lane
  BuildSpmmPlan pl;
  pl.tpw = (g.n_tiles + kSplitParts - 1) / kSplitParts;
  pl.n_chunks = (g.d_model + kWave * V - 1) / (kWave * V);
  pl.lds_bytes = static_cast<size_t>(kSplitParts) * pl.tpw * g.capacity * 8 +
                 static_cast<size_t>(kSplitParts) * V * kWave * 4;
  return pl;
}
}  // namespace

bool build_takes_spmm(const Geometry& g, int elem_bytes) {
  if (elem_bytes != 4 || g.n_rows <= 0 || route_mode(g) != 1) return false;
  const size_t row_bytes = static_cast<size_t>(g.d_ff) * 4;
  // launch_materialize's choice: slot groups for long rows of 4 or 8 slots,
  // no LDS row buffer past 64 KB
  if ((g.capacity == 4 || g.capacity == 8) && row_bytes > 20 * 1024) return false;
  if (row_bytes > 64 * 1024) return false;
  // launch_spmm_sparse's choice of the 16-range kernel for float32 (same LDS)
  const BuildSpmmPlan pl = build_spmm_plan(g);
  return g.n_rows * pl.n_chunks <= 1024 && pl.lds_bytes <= 64 * 1024;
}

hipError_t launch_materialize(const Geometry& g, int elem_bytes, const int32_t* row_map,
                              const uint8_t* flags, const void* spill, const void* full_src,
                              void* vals, uint8_t* idx, uint8_t* cnt, void* dense_values,
                              int64_t dense_cap, hipStream_t s, const RouteOut* route,
                              const BuildSpmm* sp) {
  if (g.n_rows == 0) return hipSuccess;
  if (sp != nullptr) {
    // float32, routed in the workgroup, built in LDS: 1024 threads per row
    if (!build_takes_spmm(g, elem_bytes) || route == nullptr || route->row_dense != nullptr ||
        full_src != nullptr)
      return hipErrorInvalidValue;
    const BuildSpmmPlan pl = build_spmm_plan(g);
    const size_t row_bytes = static_cast<size_t>(g.d_ff) * 4;
    const size_t lds = pl.lds_bytes > row_bytes ? pl.lds_bytes : row_bytes;
    materialize_kernel<float, true, 1, kSplitParts * kWave>
        <<<static_cast<unsigned>(g.n_rows), kSplitParts * kWave, lds, s>>>(
            g.d_ff, g.tile, g.capacity, g.n_tiles, row_map, flags,
            static_cast<const float*>(spill), nullptr, static_cast<float*>(vals), idx, cnt,
            static_cast<float*>(dense_values), dense_cap, *route, *sp, g.d_model, pl.tpw,
            pl.n_chunks);
    return hipGetLastError();
  }
  // 0: the scan's row map; 1: routed inside each workgroup; 2: counted from row_dense
  const int rmode = route == nullptr ? 0 : route->row_dense == nullptr ? 1 : 2;
  const RouteOut ro = route != nullptr ? *route : RouteOut{};
  const unsigned blocks = static_cast<unsigned>(g.n_rows);
  const size_t row_bytes = static_cast<size_t>(g.d_ff) * elem_bytes;
  // The LDS row buffer is the faster build while eight rows fit in a CU's
  // LDS (measured: 30 against 36 us for 1853 rows of 16 KB); longer rows
  // rebuild each 16-byte piece in registers from the slot groups (75
  // against 108 us for 4750 rows of 28 KB).
  if (full_src == nullptr && (g.capacity == 4 || g.capacity == 8) && row_bytes > 20 * 1024) {
    // A few rows (decode-sized batches) are latency-bound: 1024 threads per
    // row then rebuild a row in one batch of loads instead of several.
    auto run2 = [&](auto tag, auto cc, auto rm) {
      typedef decltype(tag) E;
      constexpr int RM = decltype(rm)::value;
      if (g.n_rows <= kSkinnyMaxRows)
        materialize_slots_kernel<E, decltype(cc)::value, 1024, RM><<<blocks, 1024, 0, s>>>(
            g.d_ff, g.tile, g.n_tiles, row_map, flags, static_cast<const E*>(spill),
            static_cast<E*>(vals), idx, cnt, static_cast<E*>(dense_values), dense_cap, ro);
      else
        materialize_slots_kernel<E, decltype(cc)::value, kRowThreads, RM>
            <<<blocks, kRowThreads, 0, s>>>(g.d_ff, g.tile, g.n_tiles, row_map, flags,
                                            static_cast<const E*>(spill), static_cast<E*>(vals),
                                            idx, cnt, static_cast<E*>(dense_values), dense_cap, ro);
    };
    auto run = [&](auto tag, auto cc) {
      if (rmode == 1) run2(tag, cc, std::integral_constant<int, 1>{});
      else if (rmode == 2) run2(tag, cc, std::integral_constant<int, 2>{});
      else run2(tag, cc, std::integral_constant<int, 0>{});
    };
    typedef std::integral_constant<int, 4> C4;
    typedef std::integral_constant<int, 8> C8;
    if (elem_bytes == 2) {
      if (g.capacity == 4) run(uint16_t{}, C4{}); else run(uint16_t{}, C8{});
    } else {
      if (g.capacity == 4) run(float{}, C4{}); else run(float{}, C8{});
    }
    return hipGetLastError();
  }
  const bool in_lds = full_src == nullptr && row_bytes <= 64 * 1024;
  const size_t lds = in_lds ? row_bytes : 0;
  if (rmode == 2 && full_src == nullptr) {
    // workgroups for the row blocks' lists and the dense rows only (a copy
    // from h, in twell_pack, keeps one workgroup per row: its dense rows are
    // most rows, and a workgroup that copies several rows one after another
    // was slower: 545 against 532 us at 16384 x 28672)
    const int64_t nb = (g.n_rows + kRowThreads - 1) / kRowThreads;
    const int64_t want = g.n_rows < kListedGrid ? g.n_rows : kListedGrid;
    const unsigned lblocks = static_cast<unsigned>(want > nb ? want : nb);
    auto listed = [&](auto tag, auto lds_tag) {
      typedef decltype(tag) E;
      materialize_listed_kernel<E, decltype(lds_tag)::value><<<lblocks, kRowThreads, lds, s>>>(
          g.d_ff, g.tile, g.capacity, g.n_tiles, flags, static_cast<const E*>(spill),
          static_cast<const E*>(full_src), static_cast<E*>(vals), idx, cnt,
          static_cast<E*>(dense_values), dense_cap, ro);
    };
    typedef std::integral_constant<bool, true> InLds;
    typedef std::integral_constant<bool, false> NotInLds;
    if (elem_bytes == 2) {
      if (in_lds) listed(uint16_t{}, InLds{}); else listed(uint16_t{}, NotInLds{});
    } else {
      if (in_lds) listed(float{}, InLds{}); else listed(float{}, NotInLds{});
    }
    return hipGetLastError();
  }
  auto go = [&](auto tag, auto lds_tag, auto route_tag) {
    typedef decltype(tag) E;
    materialize_kernel<E, decltype(lds_tag)::value, decltype(route_tag)::value>
        <<<blocks, kRowThreads, lds, s>>>(g.d_ff, g.tile, g.capacity, g.n_tiles, row_map, flags,
                                          static_cast<const E*>(spill),
                                          static_cast<const E*>(full_src), static_cast<E*>(vals),
                                          idx, cnt, static_cast<E*>(dense_values), dense_cap, ro,
                                          BuildSpmm{nullptr, nullptr}, 0, 0, 0);
  };
  typedef std::integral_constant<bool, true> Yes;
  typedef std::integral_constant<bool, false> No;
  auto by_route = [&](auto tag, auto lds_tag) {
    if (rmode == 1) go(tag, lds_tag, std::integral_constant<int, 1>{});
    else if (rmode == 2) go(tag, lds_tag, std::integral_constant<int, 2>{});
    else go(tag, lds_tag, std::integral_constant<int, 0>{});
  };
  auto by_lds = [&](auto tag) {
    if (in_lds) by_route(tag, Yes{}); else by_route(tag, No{});
  };
  if (elem_bytes == 2) by_lds(uint16_t{}); else by_lds(float{});
  return hipGetLastError();
}

hipError_t launch_pack_tiles(const Geometry& g, const void* h, int elem_bytes, const PackOut& out,
                             hipStream_t s) {
  const int64_t pairs = g.n_rows * g.n_tiles;
  if (pairs == 0) return hipSuccess;
  const int64_t want = (pairs + 4 * kPackAhead - 1) / (4 * kPackAhead);  // 4 waves per workgroup
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  auto go = [&](auto tag, auto epl) {
    typedef decltype(tag) E;
    pack_tiles_kernel<E, decltype(epl)::value><<<blocks, kRowThreads, 0, s>>>(
        static_cast<const E*>(h), pairs, g.d_ff, g.tile, g.capacity, g.n_tiles,
        static_cast<E*>(out.vals), out.idx, out.cnt, out.flags);
  };
  auto by_tile = [&](auto tag) {
    if (g.tile == 64) go(tag, std::integral_constant<int, 1>{});
    else if (g.tile == 128) go(tag, std::integral_constant<int, 2>{});
    else go(tag, std::integral_constant<int, 4>{});
  };
  if (elem_bytes == 2) by_tile(uint16_t{}); else by_tile(float{});
  return hipGetLastError();
}

hipError_t launch_unpack(const Geometry& g, int elem_bytes, const void* vals, const uint8_t* idx,
                         const uint8_t* cnt, const int32_t* dense_rows, const void* dense_values,
                         const int32_t* n_dense, int64_t dense_cap, void* h, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(g.n_rows);
  if (elem_bytes == 2) {
    unpack_kernel<uint16_t><<<blocks, kRowThreads, 0, s>>>(
        g.d_ff, g.tile, g.capacity, g.n_tiles, static_cast<const uint16_t*>(vals), idx, cnt,
        dense_rows, static_cast<const uint16_t*>(dense_values), n_dense, dense_cap,
        static_cast<uint16_t*>(h));
  } else {
    unpack_kernel<float><<<blocks, kRowThreads, 0, s>>>(
        g.d_ff, g.tile, g.capacity, g.n_tiles, static_cast<const float*>(vals), idx, cnt,
        dense_rows, static_cast<const float*>(dense_values), n_dense, dense_cap,
        static_cast<float*>(h));
  }
  return hipGetLastError();
}

}  // namespace twell
