// Shared by the sparse-product kernels and the kernel that runs the few-row
// sparse product beside the dense fallback's split-K partial sums: the w_down
// gather helpers and the few-row body (one workgroup of P waves per (row, XCD
// column slice), wave w gathering tiles [w * tpw, (w + 1) * tpw) of the row;
// the P partial sums meet in LDS and are added in wave order).
#pragma once

#include "common.h"
#include "kernels.h"

namespace twell {
namespace {

// bf16 products use v_dot2_f32_bf16 with one half of the value operand zero:
// y[c] += v*W[c] as a single exact-product, single-rounding step per element.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

template <int VEC>
struct WVec;
template <>
struct WVec<4> {
  uint32_t d[2];
};
template <>
struct WVec<8> {
  uint32_t d[4];
};
template <>
struct WVec<16> {
  uint32_t d[8];
};

template <int VEC>
__device__ __forceinline__ void load_wvec(WVec<VEC>& o, const uint16_t* p) {
  if constexpr (VEC == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    o.d[0] = q.x, o.d[1] = q.y;
  } else {
#pragma unroll
    for (int h = 0; h < VEC / 8; ++h) {
      const uint4 q = *reinterpret_cast<const uint4*>(p + 8 * h);
      o.d[4 * h] = q.x, o.d[4 * h + 1] = q.y, o.d[4 * h + 2] = q.z, o.d[4 * h + 3] = q.w;
    }
  }
}

template <int VEC>
__device__ __forceinline__ void dot2_row(float (&acc)[VEC], uint32_t vlo, uint32_t vhi,
                                         const WVec<VEC>& w) {
  const bf16x2_t a0 = __builtin_bit_cast(bf16x2_t, vlo);  // (v, 0)
  const bf16x2_t a1 = __builtin_bit_cast(bf16x2_t, vhi);  // (0, v)
#pragma unroll
  for (int i = 0; i < VEC / 2; ++i) {
    const bf16x2_t b = __builtin_bit_cast(bf16x2_t, w.d[i]);
    acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(a0, b, acc[2 * i], false);
    acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(a1, b, acc[2 * i + 1], false);
  }
}

// Each wave takes one row of its XCD's column slice at a time: it first
// compacts the row's live slots into a per-wave LDS list (byte offset of the
// w_down row, value) with a ballot prefix, then walks the list 8 entries at a
// time with broadcast LDS reads, keeping 8 row gathers in flight.
constexpr int kListUnroll = 8;

// Tile ranges a row is split into by the few-row sparse product: the waves
// of its own kernel, and the waves times ranges per wave of the kernel that
// runs it beside the fallback, so both sum a row the same way.
constexpr int kSplitParts = 16;

// Rows [part + parts * (vblock / 8) ...] of the sparse-row list, for
// workgroup vblock of vgrid (vblock mod 8 is the XCD; the XCD's column slice
// is xcd mod n_slices).  The row's tiles are split over P * V parts of tpw
// tiles: wave w takes parts w V .. w V + V - 1 one after the other, each
// summed on its own, and the P * V partial sums are added in part order, so
// the result does not depend on P for a given P * V.  `lists` holds
// P * tpw * C list entries, then P * V * VEC * 64 floats of partial sums.
template <int VEC, int P, int V = 1>
__device__ __forceinline__ void spmm_split_rows(
    const uint16_t* __restrict__ vals, const uint8_t* __restrict__ idx,
    const uint8_t* __restrict__ cnt, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ n_rows_dev, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ y, int64_t N, int dm, int T, int C, int nt, int n_slices, int tpw,
    uint2* lists, int64_t vblock, int64_t vgrid, DenseSkip skip = DenseSkip{nullptr, nullptr, 0}) {
  constexpr int PV = P * V;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int wslots = tpw * C;
  uint2* list = lists + wave * wslots;
  float* red = reinterpret_cast<float*>(lists + P * wslots);  // [P * V][VEC][64]
  const int xcd = static_cast<int>(vblock % 8);
  const int slice = xcd % n_slices;
  const int parts = 8 / n_slices;
  const int part = xcd / n_slices;
  const int64_t per_xcd = vgrid / 8;
  const int col = slice * (kWave * VEC) + lane * VEC;
  const char* wbase = reinterpret_cast<const char*>(w + col);
  const int64_t R = rows != nullptr ? min(static_cast<int64_t>(*n_rows_dev), N) : N;
  for (int64_t k = part + parts * (vblock / 8); k < R; k += parts * per_xcd) {
    const int64_t n = rows != nullptr ? rows[k] : k;
    if (rows == nullptr && listed_dense(n, skip.dense_rows, skip.n_dense, skip.cap)) continue;
    const int64_t s0 = n * nt * C;
    for (int vv = 0; vv < V; ++vv) {
      const int pv = wave * V + vv;
      const int t0 = pv * tpw, t1 = min(nt, t0 + tpw);
      int nnz = 0;
      for (int g = t0 * C; g < t1 * C; g += kWave) {
        const int s = g + lane;
        bool live = false;
        uint32_t off = 0, v = 0;
        if (s < t1 * C) {
          const int t = s / C;
          const int kk = s - t * C;
          if (kk < static_cast<int>(cnt[n * nt + t])) {
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
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's list is in LDS
      float acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
      for (int q = 0; q < nnz; q += kListUnroll) {
        uint2 e[kListUnroll];
        WVec<VEC> wv[kListUnroll];
#pragma unroll
        for (int u = 0; u < kListUnroll; ++u) {
          e[u] = list[min(q + u, nnz - 1)];  // past the end: reread the last entry, unused
          load_wvec<VEC>(wv[u], reinterpret_cast<const uint16_t*>(wbase + e[u].x));
        }
#pragma unroll
        for (int u = 0; u < kListUnroll; ++u)
          if (q + u < nnz) dot2_row<VEC>(acc, e[u].y, e[u].y << 16, wv[u]);
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) red[(pv * VEC + i) * kWave + lane] = acc[i];
      // the wave's list is rewritten by its next part only after its own reads
      __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    __syncthreads();
    // wave w finishes columns i = w, w + P, ... of each lane's VEC
    uint16_t* dst = y + n * dm + col;
    for (int i = wave; i < VEC; i += P) {
      float sum = 0.f;
#pragma unroll
      for (int p = 0; p < PV; ++p) sum += red[(p * VEC + i) * kWave + lane];
      dst[i] = ElemTraits<uint16_t>::from_f32(sum);
    }
    __syncthreads();  // red and the lists are reused by the next row
  }
}


// ---- few-row generic body (float32, or bf16 with a d_model the sliced
// kernel does not take): one row, one chunk of 64 lanes x 16 bytes of
// columns, its tiles cut into P * VR ranges of tpw tiles.  Wave w takes
// ranges w * VR .. w * VR + VR - 1 in turn; each range's sum goes to LDS and
// the P * VR sums are added in range order, so the result does not depend on
// how many waves share the ranges.  `lists`: P lists of tpw * C entries;
// `red`: P * VR * (16 / sizeof(E)) * 64 floats.
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

template <typename E, int P, int VR>
__device__ __forceinline__ void spmm_split_row_chunk(
    const E* __restrict__ vals, const uint8_t* __restrict__ idx, const uint8_t* __restrict__ cnt,
    int64_t n, const E* __restrict__ w, E* __restrict__ y, int dm, int T, int C, int nt, int tpw,
    int chunk, uint2* lists, float* red) {
  constexpr int V = SpmmVec<E>::N;
  typedef ElemTraits<E> Tr;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  uint2* list = lists + wave * tpw * C;
  const int col = chunk * (kWave * V) + lane * V;
  const bool live_col = col < dm;  // dm is a multiple of 8, so V columns are all in or all out
  const int64_t s0 = n * nt * C;
  for (int j = 0; j < VR; ++j) {
    const int p = wave * VR + j;
    const int t0 = p * tpw, t1 = min(nt, t0 + tpw);
    int nnz = 0;
    for (int g = t0 * C; g < t1 * C; g += kWave) {
      const int s = g + lane;
      bool live = false;
      uint32_t jj = 0;
      float v = 0.f;
      if (s < t1 * C) {
        const int t = s / C;
        if (s - t * C < static_cast<int>(cnt[n * nt + t])) {
          const int local = static_cast<int>(idx[s0 + s]);
          live = local < T;  // a malformed index is ignored rather than read out of bounds
          jj = static_cast<uint32_t>(t * T + local);
          v = Tr::to_f32(vals[s0 + s]);
        }
      }
      const uint64_t m = wave_ballot(live);
      if (live) list[nnz + popc_below(m)] = make_uint2(jj, __float_as_uint(v));
      nnz += popc64(m);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's list is in LDS
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int q = 0; q < nnz; q += kListUnroll) {
      uint2 e[kListUnroll];
      uint4 wv[kListUnroll];
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u) {
        e[u] = list[min(q + u, nnz - 1)];  // past the end: reread the last entry, unused
        wv[u] = live_col ? *reinterpret_cast<const uint4*>(w + static_cast<int64_t>(e[u].x) * dm + col)
                         : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kListUnroll; ++u)
        if (q + u < nnz) fma_row<E>(acc, __uint_as_float(e[u].y), wv[u]);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) red[(p * V + i) * kWave + lane] = acc[i];
  }
  __syncthreads();
  // wave w finishes columns i = w, w + P, ... of each lane's V
  for (int i = wave; i < V; i += P) {
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < P * VR; ++p) sum += red[(p * V + i) * kWave + lane];
    if (live_col) y[n * dm + col + i] = Tr::from_f32(sum);
  }
  __syncthreads();  // red and the lists are reused by the next row or chunk
}

}  // namespace
}  // namespace twell
