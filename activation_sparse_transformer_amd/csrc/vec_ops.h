// Wave-level vector helpers shared by the backward pass and the gated
// forward: 16-byte dot products and multiply-adds in float32 (bf16 through
// v_dot2_f32_bf16), and fixed-order sums over lane groups with DPP.
#pragma once

#include "common.h"

namespace twell {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 vec_bf16x2_t;

// sum over one 16-byte group of a[c] * b[c], in float32
template <typename E>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& b);

template <>
__device__ __forceinline__ float dot16<uint16_t>(const uint4& a, const uint4& b) {
  const uint32_t aa[4] = {a.x, a.y, a.z, a.w}, bb[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(vec_bf16x2_t, aa[i]),
                                        __builtin_bit_cast(vec_bf16x2_t, bb[i]), s, false);
  return s;
}

template <>
__device__ __forceinline__ float dot16<float>(const uint4& a, const uint4& b) {
  float s = 0.f;
  s = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), s);
  s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
  s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
  s = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
  return s;
}

// acc[i] += s * v[i] for the 16 / sizeof(E) elements of v; `s` is a value of
// the storage type (its bits in sbits).  bf16: one dot2 per element with the
// other half of the scalar operand zero, an exact product added once.
template <typename E>
__device__ __forceinline__ void axpy16(float* acc, uint32_t sbits, const uint4& v);

template <>
__device__ __forceinline__ void axpy16<uint16_t>(float* acc, uint32_t sbits, const uint4& v) {
  const vec_bf16x2_t lo = __builtin_bit_cast(vec_bf16x2_t, sbits & 0xffffu);  // (s, 0)
  const vec_bf16x2_t hi = __builtin_bit_cast(vec_bf16x2_t, sbits << 16);      // (0, s)
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const vec_bf16x2_t b = __builtin_bit_cast(vec_bf16x2_t, w[i]);
    acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(lo, b, acc[2 * i], false);
    acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, b, acc[2 * i + 1], false);
  }
}

template <>
__device__ __forceinline__ void axpy16<float>(float* acc, uint32_t sbits, const uint4& v) {
  const float s = __uint_as_float(sbits);
  acc[0] = fmaf(s, __uint_as_float(v.x), acc[0]);
  acc[1] = fmaf(s, __uint_as_float(v.y), acc[1]);
  acc[2] = fmaf(s, __uint_as_float(v.z), acc[2]);
  acc[3] = fmaf(s, __uint_as_float(v.w), acc[3]);
}

// storage bits of an fp32 value that is exactly representable in E
template <typename E>
__device__ __forceinline__ uint32_t store_bits(uint32_t f32bits) {
  return sizeof(E) == 2 ? (f32bits >> 16) : f32bits;
}

// v + (v of the lane that DPP control CTRL selects), for the rows in ROWS;
// lanes of other rows keep v.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_add(float v) {
  const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false);
  return v + __int_as_float(t);
}

// Sums of v[u] over each group of P lanes (P = 8, 16, 32, 64; groups
// aligned), valid in the group's last lane, added in a fixed order: pairs and
// quads (quad permutes), halves of rows (row_half_mirror), rows of 16
// (row_mirror), then row 0 into row 1 and row 2 into row 3 (row_bcast15) and
// rows 0-1 into row 3 (row_bcast31).  The U sums go level by level, so no
// step waits on the one before it.
template <int P, int U>
__device__ __forceinline__ void group_totals(float (&v)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = dpp_add<0xb1>(v[u]);  // quad_perm [1, 0, 3, 2]
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = dpp_add<0x4e>(v[u]);  // quad_perm [2, 3, 0, 1]
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = dpp_add<0x141>(v[u]);  // row_half_mirror
  if constexpr (P >= 16) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = dpp_add<0x140>(v[u]);  // row_mirror
  }
  if constexpr (P >= 32) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = dpp_add<0x142, 0xa>(v[u]);  // row_bcast15: rows 1, 3
  }
  if constexpr (P >= 64) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = dpp_add<0x143, 0xc>(v[u]);  // row_bcast31: rows 2, 3
  }
}

__device__ __forceinline__ uint4 keep_if(bool keep, const uint4& v) {
  return keep ? v : make_uint4(0, 0, 0, 0);
}

}  // namespace
}  // namespace twell
