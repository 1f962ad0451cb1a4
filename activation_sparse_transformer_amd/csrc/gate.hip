// The up branch of the ReLU-gated FFN, h = ReLU(x W_gate + b_gate) *
// (x W_up + b_up): once the gate's activations are packed and routed (the
// plain forward's steps 1-2 run on W_gate), the up branch is needed only where
// the gate is non-zero.  Per stored non-zero g of row n and neuron j (a TwELL
// slot of a sparse row, or a non-zero of a stored dense row),
//   u = dot(x[n], W_up[j]) + b_up[j]   (float32),
//   h = g * u                           rounded to the storage type,
// is written over g in place; the hybrid product then takes h as it takes the
// plain layer's activations.  The pages describe only the non-gated layer
// ("The Relentless Search for Efficiency in Large-Scale Language Models",
// section "The Challenge of Sparsity Ignored by GPUs": sparsity from the
// ReLU); the gated form follows the sparse LLaMA models of
// "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse Transformers Run Like
// They Were Built for Hopper", section "The Repo's Two Jobs".
#include "../../include/twell.h"
#include "common.h"
#include "kernels.h"
#include "vec_ops.h"

namespace twell {
namespace {

constexpr int kGateThreads = 256;
constexpr int kGateWaves = kGateThreads / kWave;
constexpr unsigned kGateMaxBlocks = 16384;

// Work items (one wave each, grid-stride), in one of two maps:
// * by XCD (xcd_part > 0: a row's slots split into 8 parts of xcd_part slots,
//   covering tiles, and so neurons, [x nt / 8, (x + 1) nt / 8)): the
//   workgroups on XCD x = blockIdx mod 8 take part x of every sparse row, and
//   the column chunks [x n_chunks / 8, (x + 1) n_chunks / 8) of the stored
//   dense rows, so each XCD gathers the W_up rows of about an eighth of the
//   neurons instead of all of them (measured at the 1B layer: the gated
//   forward 0.425 -> 0.41-0.43 ms; at the decode layer 0.116 -> 0.110 ms;
//   splitting each eighth into two phases, to fit the L2 better, was slower);
// * otherwise items r * P + p for r < N are slots [64 p, 64 p + 64) of sparse
//   row sparse_rows[r] (P = ceil(nt * C / 64)), and items N * P + m * n_chunks
//   + q column chunk q (64 lanes x 16 bytes) of stored dense row m.
// Rows r past n_sparse do nothing, and no wave walks a long list alone.  A
// wave lists its item's non-zeros in LDS as {neuron j, place, g bits}, then
// walks the list U entries at a time: the U gathers of W_up[j] go out
// together, the U dots are summed across the wave by DPP (into lane 63), and
// lane 63 writes the U products.  Each product is the same in either map.
template <typename E, int NVX, int U>
__global__ __launch_bounds__(kGateThreads) void gate_up_kernel(
    GateHybrid hy, const E* __restrict__ x, const E* __restrict__ w_up_t,
    const float* __restrict__ b_up, int64_t n_rows, int dm, int dff, int T, int C, int nt,
    int parts, int n_chunks, int64_t n_items, int list_len, int xcd_part) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  extern __shared__ uint4 gate_lists[];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  uint4* list = gate_lists + wave * list_len;
  const int nslots = nt * C;
  const int64_t sparse_items = n_rows * parts;
  const int64_t n_sparse = min(static_cast<int64_t>(max(*hy.n_sparse, 0)), n_rows);
  const int64_t stored = hy.cap > 0 ? min(static_cast<int64_t>(max(*hy.n_dense, 0)), hy.cap) : 0;
  E* vals = static_cast<E*>(hy.vals);
  E* dvals = static_cast<E*>(hy.dense_values);
  // the XCD map: this XCD's part, its dense chunks [qa, qb), its items
  const int xcd = static_cast<int>(blockIdx.x % 8);
  const int qa = xcd_part > 0 ? xcd * n_chunks / 8 : 0;
  const int nq = xcd_part > 0 ? (xcd + 1) * n_chunks / 8 - qa : n_chunks;
  const int64_t first = xcd_part > 0 ? static_cast<int64_t>(blockIdx.x / 8) * kGateWaves + wave
                                     : static_cast<int64_t>(blockIdx.x) * kGateWaves + wave;
  const int64_t stride = xcd_part > 0 ? static_cast<int64_t>(gridDim.x / 8) * kGateWaves
                                      : static_cast<int64_t>(gridDim.x) * kGateWaves;
  const int64_t last = xcd_part > 0 ? n_rows * (1 + nq) : n_items;
  const int64_t n_sparse_items = xcd_part > 0 ? n_rows : sparse_items;
  for (int64_t i = first; i < last; i += stride) {
    int64_t row;
    E* dst;  // the item's values: the row's slots or the dense row
    int nnz = 0;
    if (i < n_sparse_items) {  // sparse row r, slots [s0, s1)
      const int64_t r = xcd_part > 0 ? i : i / parts;
      if (r >= n_sparse) continue;
      row = hy.sparse_rows[r];
      dst = vals + row * nslots;
      const int s0 = xcd_part > 0 ? xcd * xcd_part : static_cast<int>(i % parts) * kWave;
      const int s1 = xcd_part > 0 ? s0 + xcd_part : min(s0 + kWave, nslots);
      const int s = s0 + lane;
      bool live = false;
      uint32_t j = 0, gb = 0;
      if (s < s1) {
        const int t = s / C;
        if (s - t * C < static_cast<int>(hy.cnt[row * nt + t])) {
          const int local = hy.idx[row * nslots + s];
          live = local < T;
          j = static_cast<uint32_t>(t * T + local);
          gb = static_cast<uint32_t>(__builtin_bit_cast(typename Tr::bits_t, dst[s]));
        }
      }
      const uint64_t m = wave_ballot(live);
      if (live) list[popc_below(m)] = make_uint4(j, static_cast<uint32_t>(s), gb, 0u);
      nnz = popc64(m);
    } else {  // stored dense row m, column chunk q
      const int64_t m = (i - n_sparse_items) / nq;
      if (m >= stored) break;  // items only grow: no dense item is left
      const int q = qa + static_cast<int>((i - n_sparse_items) % nq);
      const int c0 = q * (kWave * V);
      row = hy.dense_rows[m];
      dst = dvals + m * dff;
      const int c = c0 + lane * V;
      E hv[V];
      *reinterpret_cast<uint4*>(hv) =
          c < dff ? *reinterpret_cast<const uint4*>(dst + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const bool live = Tr::abs_bits(hv[e]) != 0u;
        const uint64_t mk = wave_ballot(live);
        if (live)
          list[nnz + popc_below(mk)] =
              make_uint4(static_cast<uint32_t>(c + e), static_cast<uint32_t>(c + e),
                         static_cast<uint32_t>(__builtin_bit_cast(typename Tr::bits_t, hv[e])), 0u);
        nnz += popc64(mk);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's list is in LDS
    __builtin_amdgcn_wave_barrier();
    if (nnz == 0) continue;
    // x[n] in registers
    uint4 xv[NVX];
#pragma unroll
    for (int v = 0; v < NVX; ++v) {
      const int c = (v * kWave + lane) * V;
      xv[v] = c < dm ? *reinterpret_cast<const uint4*>(x + row * dm + c) : make_uint4(0, 0, 0, 0);
    }
    for (int k = 0; k < nnz; k += U) {
      uint4 en[U];
      uint4 wv[U][NVX];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        en[u] = list[min(k + u, nnz - 1)];  // past the list: the last entry again, not written
        const E* wrow = w_up_t + static_cast<int64_t>(en[u].x) * dm;
#pragma unroll
        for (int v = 0; v < NVX; ++v) {
          // a lane past d_model reads the last group (its x is zero there)
          const int c = min((v * kWave + lane) * V, dm - V);
          wv[u][v] = *reinterpret_cast<const uint4*>(wrow + c);
        }
      }
      float d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        d[u] = 0.f;
#pragma unroll
        for (int v = 0; v < NVX; ++v) d[u] += dot16<E>(xv[v], wv[u][v]);
      }
      group_totals<kWave, U>(d);
      if (lane == kWave - 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (k + u >= nnz) break;
          const float up = d[u] + b_up[en[u].x];
          const float g = Tr::to_f32(__builtin_bit_cast(E, static_cast<typename Tr::bits_t>(en[u].z)));
          dst[en[u].y] = Tr::from_f32(g * up);
        }
      }
    }
  }
}

template <typename E, int NVX>
hipError_t launch_gate(const Geometry& g, const GateHybrid& hy, const void* x, const void* w_up_t,
                       const float* b_up, hipStream_t s) {
  constexpr int V = 16 / sizeof(E);
  constexpr int U = NVX >= 8 ? 16 / NVX : 8;
  const int n_chunks = (g.d_ff + kWave * V - 1) / (kWave * V);
  const int64_t cap = hy.cap <= 0 ? 0 : (hy.cap < g.n_rows ? hy.cap : g.n_rows);
  const int nslots = g.n_tiles * g.capacity;
  const int parts = (nslots + kWave - 1) / kWave;
  const int64_t items = g.n_rows * parts + cap * n_chunks;
  const int list_len = kWave * V;  // a 64-slot part or a dense chunk
  const size_t lds = static_cast<size_t>(kGateWaves) * list_len * sizeof(uint4);
  // the XCD map when a row's tiles split into 8 parts of at most 64 slots and
  // every XCD has a dense chunk
  const int xcd_part =
      (g.n_tiles % 8 == 0 && nslots / 8 <= kWave && n_chunks >= 8) ? nslots / 8 : 0;
  int64_t blocks = (items + kGateWaves - 1) / kGateWaves;
  if (xcd_part > 0) blocks = (blocks + 7) / 8 * 8;  // whole rounds of the 8 XCDs
  gate_up_kernel<E, NVX, U><<<static_cast<unsigned>(blocks < kGateMaxBlocks ? blocks : kGateMaxBlocks),
                              kGateThreads, lds, s>>>(
      hy, static_cast<const E*>(x), static_cast<const E*>(w_up_t), b_up, g.n_rows, g.d_model,
      g.d_ff, g.tile, g.capacity, g.n_tiles, parts, n_chunks, items, list_len, xcd_part);
  return hipGetLastError();
}

int gate_nvx(int d_model, int elem_bytes) {
  const int per = kWave * (16 / elem_bytes);
  const int vecs = (d_model + per - 1) / per;
  return vecs <= 1 ? 1 : vecs <= 2 ? 2 : vecs <= 4 ? 4 : vecs <= 8 ? 8 : vecs <= 16 ? 16 : 0;
}

}  // namespace

bool gate_supported(const Geometry& g, int elem_bytes) {
  return gate_nvx(g.d_model, elem_bytes) != 0;
}

hipError_t launch_gate_up(const Geometry& g, int elem_bytes, const GateHybrid& hy, const void* x,
                          const void* w_up_t, const float* b_up, hipStream_t s) {
  if (g.n_rows == 0) return hipSuccess;
  const int nvx = gate_nvx(g.d_model, elem_bytes);
  if (elem_bytes == 2) {
    switch (nvx) {
      case 1: return launch_gate<uint16_t, 1>(g, hy, x, w_up_t, b_up, s);
      case 2: return launch_gate<uint16_t, 2>(g, hy, x, w_up_t, b_up, s);
      case 4: return launch_gate<uint16_t, 4>(g, hy, x, w_up_t, b_up, s);
      case 8: return launch_gate<uint16_t, 8>(g, hy, x, w_up_t, b_up, s);
      case 16: return launch_gate<uint16_t, 16>(g, hy, x, w_up_t, b_up, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (nvx) {
    case 1: return launch_gate<float, 1>(g, hy, x, w_up_t, b_up, s);
    case 2: return launch_gate<float, 2>(g, hy, x, w_up_t, b_up, s);
    case 4: return launch_gate<float, 4>(g, hy, x, w_up_t, b_up, s);
    case 8: return launch_gate<float, 8>(g, hy, x, w_up_t, b_up, s);
    case 16: return launch_gate<float, 16>(g, hy, x, w_up_t, b_up, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace twell
