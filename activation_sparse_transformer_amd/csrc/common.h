// Device helpers shared by the TwELL kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twell {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ------------------------------------------------------------ storage types
// bf16 values travel as their uint16 bit patterns, fp32 as float.
template <typename E>
struct ElemTraits;

template <>
struct ElemTraits<uint16_t> {  // bfloat16
  typedef uint16_t bits_t;
  static constexpr uint32_t kAbsMask = 0x7fffu;
  __device__ static __forceinline__ float to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  // float -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
  __device__ static __forceinline__ uint16_t from_f32(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
  __device__ static __forceinline__ uint32_t abs_bits(uint16_t b) { return b & kAbsMask; }
};

template <>
struct ElemTraits<float> {
  typedef uint32_t bits_t;
  static constexpr uint32_t kAbsMask = 0x7fffffffu;
  __device__ static __forceinline__ float to_f32(float f) { return f; }
  __device__ static __forceinline__ float from_f32(float f) { return f; }
  __device__ static __forceinline__ uint32_t abs_bits(float f) {
    return __float_as_uint(f) & kAbsMask;
  }
};

// ------------------------------------------------------------ wave helpers
__device__ __forceinline__ int lane_id() { return static_cast<int>(__lane_id()); }

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return static_cast<uint64_t>(__ballot(p));
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int popc_below(uint64_t mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(mask >> 32),
      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// ------------------------------------------------------------ TwELL tile pack
// Pack one (row, tile) of h into its TwELL slots.  Called by all 64 lanes of
// a wave with uniform arguments; lane l holds the E = T/64 consecutive
// elements v[0..E) of columns [l*E, l*E+E) of the tile.
//
// Non-zeros are numbered in ascending column order with one ballot per
// element position: lane l's first non-zero lands after every non-zero of
// lanes < l (all positions) and after its own earlier positions.
//
// Writes: if count <= C, the stored values/indices in slots [0, count),
// padding (+0.0 bits, index 0) in [count, C), counts = count; if count > C,
// counts = 0 (the whole row goes dense later) and, if `spill` is given, the
// T raw elements to spill[0..T).  flag = (count > C).
template <typename E, int EPL>
__device__ __forceinline__ void pack_tile(const E (&v)[EPL], int C, E* __restrict__ vals,
                                          uint8_t* __restrict__ idx, uint8_t* __restrict__ cnt,
                                          uint8_t* __restrict__ flag, E* __restrict__ spill) {
  typedef ElemTraits<E> Tr;
  const int lane = lane_id();
  bool nz[EPL];
  int below = 0, count = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    nz[e] = Tr::abs_bits(v[e]) != 0u;
    const uint64_t m = wave_ballot(nz[e]);
    below += popc_below(m);
    count += popc64(m);
  }
  if (count <= C) {
    int p = below;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if (nz[e]) {
        vals[p] = v[e];
        idx[p] = static_cast<uint8_t>(lane * EPL + e);
        ++p;
      }
    }
    for (int s = count + lane; s < C; s += kWave) {
      vals[s] = E(0);
      idx[s] = 0;
    }
  } else if (spill != nullptr) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) spill[lane * EPL + e] = v[e];
  }
  if (lane == 0) {
    *cnt = static_cast<uint8_t>(count <= C ? count : 0);
    *flag = static_cast<uint8_t>(count > C ? 1 : 0);
  }
}

// Dispatch on T = 64 * EPL for a tile whose elements sit contiguously at
// `src` (LDS or global).  Lane l reads elements [l*EPL, l*EPL+EPL).
template <typename E>
__device__ __forceinline__ void pack_tile_from(const E* src, int T, int C, E* vals, uint8_t* idx,
                                               uint8_t* cnt, uint8_t* flag, E* spill) {
  const int lane = lane_id();
  if (T == 64) {
    E v[1] = {src[lane]};
    pack_tile<E, 1>(v, C, vals, idx, cnt, flag, spill);
  } else if (T == 128) {
    E v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) v[e] = src[lane * 2 + e];
    pack_tile<E, 2>(v, C, vals, idx, cnt, flag, spill);
  } else {
    E v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = src[lane * 4 + e];
    pack_tile<E, 4>(v, C, vals, idx, cnt, flag, spill);
  }
}

// ------------------------------------------------------------ row lists
// Whether row n is one of the stored dense rows dense_rows[0 .. min(*n_dense,
// cap)), which are strictly ascending: a binary search (cap 0: never).
__device__ __forceinline__ bool listed_dense(int64_t n, const int32_t* __restrict__ dense_rows,
                                             const int32_t* __restrict__ n_dense, int64_t cap) {
  if (cap <= 0) return false;
  const int64_t stored = min(static_cast<int64_t>(max(*n_dense, 0)), cap);
  int64_t lo = 0, hi = stored;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(dense_rows[mid]) < n) lo = mid + 1;
    else hi = mid;
  }
  return lo < stored && static_cast<int64_t>(dense_rows[lo]) == n;
}

// ------------------------------------------------------------ misc
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace twell
