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
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "spmm_split.h"

namespace twell {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

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
    const int32_t* __restrict__ rows, const int32_t* __restrict__ n_rows_dev, DenseSkip skip,
    const E* __restrict__ w, E* __restrict__ y, int64_t N, int dm, int T, int C, int nt,
    int n_chunks) {
  constexpr int V = SpmmVec<E>::N;
  typedef ElemTraits<E> Tr;
  const int lane = lane_id();
  const int64_t R = rows != nullptr ? min(static_cast<int64_t>(*n_rows_dev), N) : N;
  const int64_t items = R * n_chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nslots = nt * C;
  for (int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
       item < items; item += stride) {
    const int chunk = static_cast<int>(item / R);
    const int64_t k = item % R;
    const int64_t n = rows != nullptr ? rows[k] : k;  // a listed (sparse) row, or every row
    if (rows == nullptr && listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
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

// ---------------------------------------------------------------- XCD-sliced
// Workgroups are dealt round-robin to the 8 XCDs, and each XCD has its own
// L2.  Here XCD x owns column slice (x mod n_slices) of w_down and y, so the
// rows it gathers stay in its L2 (d_model/8 columns x d_ff rows).  Each wave
// takes one row at a time over its slice: VEC consecutive columns per lane.
// bf16 products use v_dot2_f32_bf16 with one half of the value operand zero:
// y[c] += v*W[c] as a single exact-product, single-rounding step per element.

// The row's live slots into the wave's LDS list in ascending slot order
// (byte offset of the w_down row, value); returns their number.  SPL > 0: the
// row has exactly 64 * SPL slots and lane l takes slots [l * SPL, l * SPL +
// SPL), all loaded in one round (one index load and one value load of SPL
// elements when SPL is 4 or 8), and a 4-ballot prefix sum of the lanes' live
// counts places them; SPL == 0: 64 slots per round for any slot count.
template <int SPL>
__device__ __forceinline__ int compact_row(const uint16_t* __restrict__ vals,
                                           const uint8_t* __restrict__ idx,
                                           const uint8_t* __restrict__ cnt, int64_t n, int nt,
                                           int C, int T, int dm, int nslots, uint2* list) {
  const int lane = lane_id();
  const int64_t s0 = n * nslots;
  if constexpr (SPL > 0) {
    uint8_t li[SPL];
    uint16_t lv[SPL];
    uint8_t lc[SPL];
    const int sb = lane * SPL;
    if constexpr (SPL == 4) {
      *reinterpret_cast<uint32_t*>(li) = *reinterpret_cast<const uint32_t*>(idx + s0 + sb);
      *reinterpret_cast<uint2*>(lv) = *reinterpret_cast<const uint2*>(vals + s0 + sb);
    } else if constexpr (SPL == 8) {
      *reinterpret_cast<uint2*>(li) = *reinterpret_cast<const uint2*>(idx + s0 + sb);
      *reinterpret_cast<uint4*>(lv) = *reinterpret_cast<const uint4*>(vals + s0 + sb);
    } else {
#pragma unroll
      for (int i = 0; i < SPL; ++i) li[i] = idx[s0 + sb + i], lv[i] = vals[s0 + sb + i];
    }
    if (C % SPL == 0) {  // the lane's slots are in one tile: one count
      const uint8_t c1 = cnt[n * nt + sb / C];
#pragma unroll
      for (int i = 0; i < SPL; ++i) lc[i] = c1;
    } else {
#pragma unroll
      for (int i = 0; i < SPL; ++i) lc[i] = cnt[n * nt + (sb + i) / C];
    }
    bool live[SPL];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int s = sb + i;
      live[i] = (s - (s / C) * C) < static_cast<int>(lc[i]) && static_cast<int>(li[i]) < T;
      mine += live[i];
    }
    int before = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // mine <= SPL <= 8
      const uint64_t m = wave_ballot((mine >> b) & 1);
      before += popc_below(m) << b;
      total += popc64(m) << b;
    }
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      if (live[i]) {
        const int s = sb + i;
        const int t = s / C;
        list[before++] = make_uint2(
            static_cast<uint32_t>(t * T + li[i]) * static_cast<uint32_t>(dm) * 2u, lv[i]);
      }
    }
    return total;
  } else {
    int nnz = 0;
    for (int g = 0; g < nslots; g += kWave) {
      const int s = g + lane;
      bool live = false;
      uint32_t off = 0, v = 0;
      if (s < nslots) {
        const int t = s / C;
        const int k = s - t * C;
        if (k < static_cast<int>(cnt[n * nt + t])) {
          const int local = static_cast<int>(idx[s0 + s]);
          live = local < T;  // a malformed index is ignored rather than read out of bounds
          off = static_cast<uint32_t>(t * T + local) * static_cast<uint32_t>(dm) * 2u;
          v = vals[s0 + s];
        }
      }
      const uint64_t m = wave_ballot(live);
      if (live) list[nnz + popc_below(m)] = make_uint2(off, v);
      nnz += popc64(m);
    }
    return nnz;
  }
}

template <int VEC, int SPL>
__global__ __launch_bounds__(kThreads) void spmm_list_bf16_kernel(
    const uint16_t* __restrict__ vals, const uint8_t* __restrict__ idx,
    const uint8_t* __restrict__ cnt, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows_dev, DenseSkip skip, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ y, int64_t N, int dm, int T, int C, int nt, int n_slices) {
  extern __shared__ uint2 spmm_lists[];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int nslots = nt * C;
  uint2* list = spmm_lists + wave * nslots;
  const int xcd = blockIdx.x % 8;
  const int slice = xcd % n_slices;
  const int parts = 8 / n_slices;  // XCDs sharing this slice split its rows
  const int part = xcd / n_slices;
  const int64_t per_xcd_waves = static_cast<int64_t>(gridDim.x / 8) * kWavesPerBlock;
  const int64_t wid = static_cast<int64_t>(blockIdx.x / 8) * kWavesPerBlock + wave;
  const int col = slice * (kWave * VEC) + lane * VEC;
  const char* wbase = reinterpret_cast<const char*>(w + col);
  const int64_t R = rows != nullptr ? min(static_cast<int64_t>(*n_rows_dev), N) : N;
  for (int64_t k = part + parts * wid; k < R; k += parts * per_xcd_waves) {
    const int64_t n = rows != nullptr ? rows[k] : k;
    if (rows == nullptr && listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
    const int nnz = compact_row<SPL>(vals, idx, cnt, n, nt, C, T, dm, nslots, list);
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
    if constexpr (VEC == 4) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
    } else {
#pragma unroll
      for (int h = 0; h < VEC / 8; ++h)
        *reinterpret_cast<uint4*>(dst + 8 * h) =
            make_uint4(out[4 * h], out[4 * h + 1], out[4 * h + 2], out[4 * h + 3]);
    }
  }
}

// Few rows (decode-sized batches): one workgroup of P waves per (row, XCD
// column slice), wave w taking tiles [w * tpw, (w + 1) * tpw) of the row, so
// the row's gathers run P ways in parallel instead of one after the other.
// The P partial sums meet in LDS and are added in wave order.
template <int VEC, int P>
__global__ __launch_bounds__(P * kWave) void spmm_split_bf16_kernel(
    const uint16_t* __restrict__ vals, const uint8_t* __restrict__ idx,
    const uint8_t* __restrict__ cnt, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows_dev, DenseSkip skip, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ y, int64_t N, int dm, int T, int C, int nt, int n_slices, int tpw) {
  extern __shared__ uint2 spmm_lists[];
  spmm_split_rows<VEC, P>(vals, idx, cnt, rows, n_rows_dev, w, y, N, dm, T, C, nt, n_slices, tpw,
                          spmm_lists, blockIdx.x, gridDim.x, skip);
}

// Few rows, float32 (or a d_model the XCD-sliced kernel does not take): one
// workgroup of P waves per (row, chunk of 64 lanes x 16 bytes of columns),
// wave w gathering tiles [w * tpw, (w + 1) * tpw) of the row; the P partial
// sums meet in LDS and are added in wave order (spmm_split_row_chunk).
template <typename E, int P>
__global__ __launch_bounds__(P * kWave) void spmm_split_kernel(
    const E* __restrict__ vals, const uint8_t* __restrict__ idx, const uint8_t* __restrict__ cnt,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ n_rows_dev, DenseSkip skip,
    const E* __restrict__ w, E* __restrict__ y, int64_t N, int dm, int T, int C, int nt,
    int n_chunks, int tpw) {
  extern __shared__ uint2 spmm_lists[];
  float* red = reinterpret_cast<float*>(spmm_lists + P * tpw * C);  // [P][V][64]
  const int64_t R = rows != nullptr ? min(static_cast<int64_t>(*n_rows_dev), N) : N;
  for (int64_t k = blockIdx.x; k < R; k += gridDim.x) {
    const int64_t n = rows != nullptr ? rows[k] : k;
    if (rows == nullptr && listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
    spmm_split_row_chunk<E, P, 1>(vals, idx, cnt, n, w, y, dm, T, C, nt, tpw, blockIdx.y,
                                  spmm_lists, red);
  }
}

// The one place the sparse product's kernel is chosen (launch_spmm_sparse,
// and the kernels that run its few-row form inside another launch).
enum class SpmmKind {
  kSplitSliced,  // bf16, few rows: 16 waves per (row, XCD column slice)
  kListSliced,   // bf16: one wave per (row, XCD column slice), slot list in LDS
  kSplitChunk,   // few rows, other widths or float32: 16 waves per (row, 64-lane chunk)
  kWaveChunk,    // anything else: one wave per (row, 64-lane chunk)
};
struct SpmmPlan {
  SpmmKind kind;
  int n_slices, vec;  // sliced kinds: column slices, bf16 per lane
  int n_chunks;       // chunk kinds: 64-lane column chunks
  int tpw;            // split kinds: tiles per range
  int spl;            // kListSliced: slots per lane when a row's slots fill whole waves, else 0
  unsigned blocks;
  size_t lds_bytes;
};

SpmmPlan spmm_plan(const Geometry& g, int elem_bytes) {
  SpmmPlan p{};
  const int V = elem_bytes == 2 ? SpmmVec<uint16_t>::N : SpmmVec<float>::N;
  p.n_chunks = (g.d_model + kWave * V - 1) / (kWave * V);
  constexpr int P = kSplitParts;
  p.tpw = (g.n_tiles + P - 1) / P;
  const size_t split_lists = static_cast<size_t>(P) * p.tpw * g.capacity * 8;
  if (elem_bytes == 2 && g.d_model % 512 == 0) {
    // Column slices of 64 lanes x 8 bf16 (x 16 when d_model/8 needs it), one
    // per XCD or shared by 2, 4, 8 XCDs; slot lists must fit in LDS, and
    // w_down byte offsets in 32 bits.
    const int ns = g.d_model / 512;
    if (ns == 1 || ns == 2 || ns == 4 || ns == 8) p.n_slices = ns, p.vec = 8;
    else if (ns == 16) p.n_slices = 8, p.vec = 16;
    const size_t list_bytes = static_cast<size_t>(kWavesPerBlock) * g.n_tiles * g.capacity * 8;
    const bool offsets_fit = static_cast<int64_t>(g.d_ff) * g.d_model * 2 < (int64_t{1} << 32);
    if (p.n_slices > 0 && list_bytes <= 64 * 1024 && offsets_fit) {
      const int64_t rows_per_xcd = (g.n_rows + (8 / p.n_slices) - 1) / (8 / p.n_slices);
      const size_t split_bytes =
          split_lists + static_cast<size_t>(P) * p.vec * kWave * 4;
      if (g.n_rows * p.n_slices <= 1024 && split_bytes <= 64 * 1024) {
        p.kind = SpmmKind::kSplitSliced;
        p.blocks = static_cast<unsigned>(8 * rows_per_xcd);
        p.lds_bytes = split_bytes;
        return p;
      }
      const int64_t wg_per_xcd = (rows_per_xcd + kWavesPerBlock - 1) / kWavesPerBlock;
      const int nslots = g.n_tiles * g.capacity;
      const int spl = nslots % kWave == 0 ? nslots / kWave : 0;
      p.kind = SpmmKind::kListSliced;
      p.spl = (spl == 2 || spl == 4 || spl == 8) ? spl : 0;
      p.blocks = static_cast<unsigned>(8 * (wg_per_xcd < 512 ? wg_per_xcd : 512));
      p.lds_bytes = list_bytes;
      return p;
    }
  }
  const size_t split_bytes = split_lists + static_cast<size_t>(P) * V * kWave * 4;
  if (g.n_rows * p.n_chunks <= 1024 && split_bytes <= 64 * 1024) {
    p.kind = SpmmKind::kSplitChunk;
    p.blocks = static_cast<unsigned>(g.n_rows);
    p.lds_bytes = split_bytes;
    return p;
  }
  const int64_t want = (g.n_rows * p.n_chunks + kWavesPerBlock - 1) / kWavesPerBlock;
  p.kind = SpmmKind::kWaveChunk;
  p.blocks = static_cast<unsigned>(want < 16384 ? want : 16384);
  p.lds_bytes = 0;
  return p;
}

}  // namespace

bool spmm_split_plan(const Geometry& g, int waves, int parts_per_wave, SpmmSplitPlan* plan) {
  if (g.n_rows <= 0) return false;
  const SpmmPlan p = spmm_plan(g, 2);
  if (p.kind != SpmmKind::kSplitSliced) return false;
  // the same kSplitParts tile ranges, taken by `waves` waves of parts_per_wave each
  plan->n_slices = p.n_slices;
  plan->vec = p.vec;
  plan->tpw = p.tpw;
  plan->blocks = p.blocks;
  plan->lds_bytes = static_cast<size_t>(waves) * p.tpw * g.capacity * 8 +
                    static_cast<size_t>(waves) * parts_per_wave * p.vec * kWave * 4;
  return waves * parts_per_wave == kSplitParts;
}

hipError_t launch_spmm_sparse(const Geometry& g, int elem_bytes, const void* vals,
                              const uint8_t* idx, const uint8_t* cnt, const int32_t* rows,
                              const int32_t* n_rows_dev, const DenseSkip* skip_in,
                              const void* w_down, void* y, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const DenseSkip skip = (rows == nullptr && skip_in != nullptr) ? *skip_in
                                                                  : DenseSkip{nullptr, nullptr, 0};
  const SpmmPlan p = spmm_plan(g, elem_bytes);
  constexpr int P = kSplitParts;
  if (elem_bytes == 2) {
    const uint16_t* v16 = static_cast<const uint16_t*>(vals);
    const uint16_t* w16 = static_cast<const uint16_t*>(w_down);
    uint16_t* y16 = static_cast<uint16_t*>(y);
    switch (p.kind) {
      case SpmmKind::kSplitSliced:
        if (p.vec == 8)
          spmm_split_bf16_kernel<8, P><<<p.blocks, P * kWave, p.lds_bytes, s>>>(
              v16, idx, cnt, rows, n_rows_dev, skip, w16, y16, g.n_rows, g.d_model, g.tile,
              g.capacity, g.n_tiles, p.n_slices, p.tpw);
        else
          spmm_split_bf16_kernel<16, P><<<p.blocks, P * kWave, p.lds_bytes, s>>>(
              v16, idx, cnt, rows, n_rows_dev, skip, w16, y16, g.n_rows, g.d_model, g.tile,
              g.capacity, g.n_tiles, p.n_slices, p.tpw);
        break;
      case SpmmKind::kListSliced: {
        auto go = [&](auto vc, auto sc) {
          spmm_list_bf16_kernel<decltype(vc)::value, decltype(sc)::value>
              <<<p.blocks, kThreads, p.lds_bytes, s>>>(v16, idx, cnt, rows, n_rows_dev, skip, w16,
                                                       y16, g.n_rows, g.d_model, g.tile,
                                                       g.capacity, g.n_tiles, p.n_slices);
        };
        auto by_spl = [&](auto vc) {
          if (p.spl == 2) go(vc, std::integral_constant<int, 2>{});
          else if (p.spl == 4) go(vc, std::integral_constant<int, 4>{});
          else if (p.spl == 8) go(vc, std::integral_constant<int, 8>{});
          else go(vc, std::integral_constant<int, 0>{});
        };
        if (p.vec == 8) by_spl(std::integral_constant<int, 8>{});
        else by_spl(std::integral_constant<int, 16>{});
        break;
      }
      case SpmmKind::kSplitChunk:
        spmm_split_kernel<uint16_t, P><<<dim3(p.blocks, p.n_chunks), P * kWave, p.lds_bytes, s>>>(
            v16, idx, cnt, rows, n_rows_dev, skip, w16, y16, g.n_rows, g.d_model, g.tile,
            g.capacity, g.n_tiles, p.n_chunks, p.tpw);
        break;
      case SpmmKind::kWaveChunk:
        spmm_sparse_kernel<uint16_t><<<p.blocks, kThreads, 0, s>>>(
            v16, idx, cnt, rows, n_rows_dev, skip, w16, y16, g.n_rows, g.d_model, g.tile,
            g.capacity, g.n_tiles, p.n_chunks);
        break;
    }
  } else {
    const float* v32 = static_cast<const float*>(vals);
    const float* w32 = static_cast<const float*>(w_down);
    float* y32 = static_cast<float*>(y);
    if (p.kind == SpmmKind::kSplitChunk)
      spmm_split_kernel<float, P><<<dim3(p.blocks, p.n_chunks), P * kWave, p.lds_bytes, s>>>(
          v32, idx, cnt, rows, n_rows_dev, skip, w32, y32, g.n_rows, g.d_model, g.tile,
          g.capacity, g.n_tiles, p.n_chunks, p.tpw);
    else
      spmm_sparse_kernel<float><<<p.blocks, kThreads, 0, s>>>(
          v32, idx, cnt, rows, n_rows_dev, skip, w32, y32, g.n_rows, g.d_model, g.tile,
          g.capacity, g.n_tiles, p.n_chunks);
  }
  return hipGetLastError();
}

}  // namespace twell
