// The layer's training step: gradients of L = sum(y * dy) from the stored
// hybrid activations ("Sparser, Faster, Lighter Transformer Language Models
// (Sakana AI + NVIDIA)", TL;DR: the format serves training as well as
// inference; "Nvidia and Sakana make LLMs 30% faster by doing less math",
// section "More speed, less power, zero quality loss": faster training with
// lower peak memory).  The ReLU passes gradient exactly where the stored
// activation is non-zero, so every gradient is read from h's non-zeros:
//
//   dz      = dy W_down^T at the non-zeros of h (a sampled product), in the
//             TwELL slots of the sparse rows and at the non-zeros of the
//             stored dense rows, rounded to the storage type;
//   dW_down = h^T dy, dW_up^T = dz^T x, db = sum of dz: per neuron j, sums
//             over the rows where h[., j] != 0, read from column lists of the
//             row-wise hybrid.  The lists are built without atomics on their
//             order: a bitmap of (neuron, row) (atomic OR, order-free), per-
//             neuron prefix counts of its 64-row words, and then each entry's
//             place is its row's rank, so every sum runs in ascending row
//             order and the result does not depend on scheduling;
//   dx      = dz W_up^T: the hybrid product (TwELL gather for the sparse
//             rows, dense fallback GEMM for the stored dense rows) with dz's
//             values in h's slots.
#include <type_traits>

#include "../../include/twell.h"
#include "common.h"
#include "kernels.h"

namespace twell {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bwd_bf16x2_t;

constexpr int kBwdThreads = 256;
constexpr int kBwdWaves = kBwdThreads / kWave;
constexpr int kBwdScanThreads = 1024;
constexpr unsigned kBwdMaxBlocks = 65536;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// sum over one 16-byte group of a[c] * b[c], in float32
template <typename E>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& b);

template <>
__device__ __forceinline__ float dot16<uint16_t>(const uint4& a, const uint4& b) {
  const uint32_t aa[4] = {a.x, a.y, a.z, a.w}, bb[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bwd_bf16x2_t, aa[i]),
                                        __builtin_bit_cast(bwd_bf16x2_t, bb[i]), s, false);
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

// Dots of row a with up to four rows b[0 .. k) (length dm), over the wave:
// lane l takes 16-byte groups l, l + 64, ...; the rows' loads go out
// together.  Rows u >= k are not read and give 0.
template <typename E>
__device__ __forceinline__ void wave_dots4(const E* __restrict__ a, const E* const (&b)[4], int k,
                                           int dm, float (&out)[4]) {
  constexpr int V = 16 / sizeof(E);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = lane_id() * V; c < dm; c += kWave * V) {
    const uint4 av = *reinterpret_cast<const uint4*>(a + c);
    uint4 bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      bv[u] = u < k ? *reinterpret_cast<const uint4*>(b[u] + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += dot16<E>(av, bv[u]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) out[u] = wave_sum(acc[u]);
}

// Index of row n among the stored dense rows (ascending), or -1.
__device__ __forceinline__ int64_t dense_index(int64_t n, const int32_t* __restrict__ dense_rows,
                                               int64_t stored) {
  int64_t lo = 0, hi = stored;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (static_cast<int64_t>(dense_rows[mid]) < n) lo = mid + 1;
    else hi = mid;
  }
  return lo < stored && dense_rows[lo] == n ? lo : -1;
}

__device__ __forceinline__ int64_t stored_dense(const BwdHybrid& hy) {
  if (hy.cap <= 0) return 0;
  return min(static_cast<int64_t>(max(*hy.n_dense, 0)), hy.cap);
}

// Work items of the row-wise passes: items [0, N) are token rows (their TwELL
// slots; a row listed among the stored dense rows is skipped), items
// N + m * n_chunks + q are column chunk q (64 lanes x 16 bytes) of stored
// dense row m.  Item i is taken by wave i of a grid-stride loop; dense items
// past the stored rows end the loop (they only grow with i).
struct Items {
  int64_t n_rows;
  int n_chunks;
  int64_t total;
};

__device__ __forceinline__ int64_t first_item() {
  return static_cast<int64_t>(blockIdx.x) * kBwdWaves + threadIdx.x / kWave;
}
__device__ __forceinline__ int64_t item_stride() {
  return static_cast<int64_t>(gridDim.x) * kBwdWaves;
}

// 1. dz at the non-zeros of h.  A token row's live slots get dot(dy[n],
// W_down[j]) in the same slot of dz_vals (padding slots 0); a dense chunk
// gets the dot at each non-zero of the stored row (0 elsewhere) in dz_dense.
// Four dots share each pass over d_model.
template <typename E>
__global__ __launch_bounds__(kBwdThreads) void bwd_dz_kernel(
    BwdHybrid hy, Items it, const E* __restrict__ dy, const E* __restrict__ w_down,
    E* __restrict__ dz_vals, E* __restrict__ dz_dense, int dm, int dff, int T, int C, int nt) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  const int lane = lane_id();
  const int nslots = nt * C;
  const int64_t stored = stored_dense(hy);
  for (int64_t i = first_item(); i < it.total; i += item_stride()) {
    if (i >= it.n_rows) {
      const int64_t m = (i - it.n_rows) / it.n_chunks;
      if (m >= stored) break;
      const int base = static_cast<int>((i - it.n_rows) % it.n_chunks) * (kWave * V);
      const int col = base + lane * V;
      const E* a = dy + static_cast<int64_t>(hy.dense_rows[m]) * dm;
      E hv[V], ov[V];
      *reinterpret_cast<uint4*>(hv) =
          col < dff ? *reinterpret_cast<const uint4*>(static_cast<const E*>(hy.dense_values) +
                                                      m * dff + col)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < V; ++e) ov[e] = E(0);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        uint64_t msk = wave_ballot(Tr::abs_bits(hv[e]) != 0u);
        while (msk != 0) {
          int L[4];
          const E* b[4];
          int k = 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            L[u] = -1;
            b[u] = w_down;
            if (msk != 0) {
              L[u] = __builtin_ctzll(msk);
              msk &= msk - 1;
              b[u] = w_down + static_cast<int64_t>(base + L[u] * V + e) * dm;
              ++k;
            }
          }
          float d[4];
          wave_dots4<E>(a, b, k, dm, d);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (lane == L[u]) ov[e] = Tr::from_f32(d[u]);
        }
      }
      if (col < dff)
        *reinterpret_cast<uint4*>(dz_dense + m * dff + col) = *reinterpret_cast<const uint4*>(ov);
      continue;
    }
    const int64_t n = i;
    if (stored > 0 && dense_index(n, hy.dense_rows, stored) >= 0) continue;
    const E* a = dy + n * dm;
    const uint8_t* irow = hy.idx + n * nslots;
    for (int g = 0; g < nslots; g += kWave) {
      const int s = g + lane;
      bool live = false;
      int j = 0;
      if (s < nslots) {
        const int t = s / C;
        if (s - t * C < static_cast<int>(hy.cnt[n * nt + t])) {
          const int local = irow[s];
          live = local < T;  // an index past the tile is not a position of h
          j = t * T + local;
        }
      }
      E ov = E(0);
      uint64_t msk = wave_ballot(live);
      while (msk != 0) {
        int L[4];
        const E* b[4];
        int k = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          L[u] = -1;
          b[u] = w_down;
          if (msk != 0) {
            L[u] = __builtin_ctzll(msk);
            msk &= msk - 1;
            b[u] = w_down + static_cast<int64_t>(__shfl(j, L[u], kWave)) * dm;
            ++k;
          }
        }
        float d[4];
        wave_dots4<E>(a, b, k, dm, d);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (lane == L[u]) ov = Tr::from_f32(d[u]);
      }
      if (s < nslots) dz_vals[n * nslots + s] = ov;
    }
  }
}

// Visit every non-zero (neuron j, row n) of h with its slot's h and dz.
// MARK sets bit n % 64 of bits[j][n / 64]; otherwise the entry goes to its
// place offsets[j] + lpre[j][n / 64] + (bits of that word below n % 64).
template <typename E, bool MARK>
__global__ __launch_bounds__(kBwdThreads) void bwd_columns_kernel(
    BwdHybrid hy, Items it, const E* __restrict__ dz_vals, const E* __restrict__ dz_dense, int dff,
    int T, int C, int nt, int64_t n_words, unsigned long long* __restrict__ bits,
    const int32_t* __restrict__ lpre, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ ent_row, float2* __restrict__ ent_hz) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  const int lane = lane_id();
  const int nslots = nt * C;
  const int64_t stored = stored_dense(hy);
  auto visit = [&](int j, int64_t n, E h, E dz) {
    const int64_t w = static_cast<int64_t>(j) * n_words + (n >> 6);
    const unsigned long long bit = 1ull << (n & 63);
    if constexpr (MARK) {
      atomicOr(bits + w, bit);
    } else {
      const int pos = offsets[j] + lpre[w] + __popcll(bits[w] & (bit - 1));
      ent_row[pos] = static_cast<int32_t>(n);
      ent_hz[pos] = make_float2(Tr::to_f32(h), Tr::to_f32(dz));
    }
  };
  for (int64_t i = first_item(); i < it.total; i += item_stride()) {
    if (i >= it.n_rows) {
      const int64_t m = (i - it.n_rows) / it.n_chunks;
      if (m >= stored) break;
      const int col = static_cast<int>((i - it.n_rows) % it.n_chunks) * (kWave * V) + lane * V;
      if (col >= dff) continue;
      const int64_t n = hy.dense_rows[m];
      E hv[V], zv[V];
      *reinterpret_cast<uint4*>(hv) =
          *reinterpret_cast<const uint4*>(static_cast<const E*>(hy.dense_values) + m * dff + col);
      if constexpr (!MARK)
        *reinterpret_cast<uint4*>(zv) = *reinterpret_cast<const uint4*>(dz_dense + m * dff + col);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (Tr::abs_bits(hv[e]) != 0u) visit(col + e, n, hv[e], MARK ? E(0) : zv[e]);
      continue;
    }
    const int64_t n = i;
    if (stored > 0 && dense_index(n, hy.dense_rows, stored) >= 0) continue;
    const E* vrow = static_cast<const E*>(hy.vals) + n * nslots;
    const uint8_t* irow = hy.idx + n * nslots;
    for (int s = lane; s < nslots; s += kWave) {
      const int t = s / C;
      if (s - t * C < static_cast<int>(hy.cnt[n * nt + t])) {
        const int local = irow[s];
        if (local < T) visit(t * T + local, n, vrow[s], MARK ? E(0) : dz_vals[n * nslots + s]);
      }
    }
  }
}

__global__ __launch_bounds__(kBwdThreads) void bwd_zero_kernel(uint32_t* __restrict__ p,
                                                               int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBwdThreads)
    p[i] = 0u;
}

// Per neuron j (one wave each): lpre[j][b] = set bits of words [0, b) of
// bits[j], and ncount[j] = all its set bits.
__global__ __launch_bounds__(kBwdThreads) void bwd_word_prefix_kernel(
    const unsigned long long* __restrict__ bits, int64_t n_words, int dff,
    int32_t* __restrict__ lpre, int32_t* __restrict__ ncount) {
  const int lane = lane_id();
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kBwdWaves + threadIdx.x / kWave;
  if (j >= dff) return;
  const unsigned long long* row = bits + j * n_words;
  int32_t* out = lpre + j * n_words;
  int run = 0;
  for (int64_t b0 = 0; b0 < n_words; b0 += kWave) {
    const int64_t b = b0 + lane;
    const int c = b < n_words ? __popcll(row[b]) : 0;
    int v = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(v, o, kWave);
      if (lane >= o) v += u;
    }
    if (b < n_words) out[b] = run + v - c;
    run += __shfl(v, kWave - 1, kWave);
  }
  if (lane == 0) ncount[j] = run;
}

// offsets[j] = ncount[0] + ... + ncount[j - 1] for j in [0, dff], one workgroup.
__global__ __launch_bounds__(kBwdScanThreads) void bwd_offsets_kernel(
    const int32_t* __restrict__ ncount, int dff, int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[kBwdScanThreads / kWave];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int per = (dff + kBwdScanThreads - 1) / kBwdScanThreads;
  const int j0 = min(dff, tid * per), j1 = min(dff, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) local += ncount[j];
  int v = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = v;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kBwdScanThreads / kWave; ++w) {
    before += w < wave ? wave_tot[w] : 0;
    total += wave_tot[w];
  }
  int run = before + v - local;
  for (int j = j0; j < j1; ++j) {
    offsets[j] = run;
    run += ncount[j];
  }
  if (tid == 0) offsets[dff] = total;
}

// dW_down[j] = sum h * dy[row], dW_up^T[j] = sum dz * x[row], db[j] = sum dz,
// over neuron j's entries in ascending row order: one wave per (neuron,
// column chunk of 64 lanes x 16 bytes), four entries' rows in flight.
template <typename E>
__global__ __launch_bounds__(kBwdThreads) void bwd_weights_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ ent_row,
    const float2* __restrict__ ent_hz, const E* __restrict__ x, const E* __restrict__ dy, int dff,
    int dm, int n_chunks, float* __restrict__ dw_up_t, float* __restrict__ db,
    float* __restrict__ dw_down) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  const int lane = lane_id();
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kBwdWaves + threadIdx.x / kWave;
  if (item >= static_cast<int64_t>(dff) * n_chunks) return;
  const int j = static_cast<int>(item / n_chunks), chunk = static_cast<int>(item % n_chunks);
  const int col = chunk * (kWave * V) + lane * V;
  const bool live_col = col < dm;
  float ad[V], au[V];
#pragma unroll
  for (int i = 0; i < V; ++i) ad[i] = 0.f, au[i] = 0.f;
  float sdz = 0.f;
  const int b = offsets[j], L = offsets[j + 1] - b;
  for (int r = 0; r < L; r += 4) {
    uint4 yv[4], xv[4];
    float2 hz[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = b + min(r + u, L - 1);  // past the end: the last again, not used
      const int64_t row = ent_row[e];
      hz[u] = ent_hz[e];
      yv[u] = live_col ? *reinterpret_cast<const uint4*>(dy + row * dm + col) : make_uint4(0, 0, 0, 0);
      xv[u] = live_col ? *reinterpret_cast<const uint4*>(x + row * dm + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r + u >= L) break;
      E ye[V], xe[V];
      *reinterpret_cast<uint4*>(ye) = yv[u];
      *reinterpret_cast<uint4*>(xe) = xv[u];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        ad[i] = fmaf(hz[u].x, Tr::to_f32(ye[i]), ad[i]);
        au[i] = fmaf(hz[u].y, Tr::to_f32(xe[i]), au[i]);
      }
      sdz += hz[u].y;
    }
  }
  if (live_col) {
    float* pd = dw_down + static_cast<int64_t>(j) * dm + col;
    float* pu = dw_up_t + static_cast<int64_t>(j) * dm + col;
#pragma unroll
    for (int q = 0; q < V; q += 4) {
      *reinterpret_cast<float4*>(pd + q) = make_float4(ad[q], ad[q + 1], ad[q + 2], ad[q + 3]);
      *reinterpret_cast<float4*>(pu + q) = make_float4(au[q], au[q + 1], au[q + 2], au[q + 3]);
    }
  }
  if (chunk == 0 && lane == 0) db[j] = sdz;
}

unsigned grid_for(int64_t waves) {
  const int64_t blocks = (waves + kBwdWaves - 1) / kBwdWaves;
  return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > kBwdMaxBlocks ? kBwdMaxBlocks : blocks));
}

hipError_t zero_words(void* p, int64_t words, hipStream_t s) {
  if (words <= 0) return hipSuccess;
  const int64_t blocks = (words + kBwdThreads - 1) / kBwdThreads;
  bwd_zero_kernel<<<static_cast<unsigned>(blocks > kBwdMaxBlocks ? kBwdMaxBlocks : blocks),
                    kBwdThreads, 0, s>>>(static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

int64_t clamp_cap(const Geometry& g, int64_t dense_cap) {
  return dense_cap <= 0 ? 0 : (dense_cap < g.n_rows ? dense_cap : g.n_rows);
}

}  // namespace

int64_t bwd_max_entries(const Geometry& g, int64_t dense_cap) {
  return g.n_rows * g.n_tiles * g.capacity + clamp_cap(g, dense_cap) * g.d_ff;
}

BwdWorkspace bwd_carve(const Geometry& g, int elem_bytes, int64_t dense_cap, void* ws) {
  const size_t cap = static_cast<size_t>(clamp_cap(g, dense_cap));
  const size_t slots = static_cast<size_t>(g.n_rows) * g.n_tiles * g.capacity;
  const size_t words = static_cast<size_t>(g.d_ff) * static_cast<size_t>((g.n_rows + 63) / 64);
  const size_t ents = static_cast<size_t>(bwd_max_entries(g, dense_cap));
  uint8_t* p = static_cast<uint8_t*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* q = p == nullptr ? nullptr : p + off;
    off += align256(bytes);
    return q;
  };
  BwdWorkspace w{};
  w.dz_vals = take(slots * elem_bytes);
  w.dz_dense = take(cap * g.d_ff * elem_bytes);
  w.bits = static_cast<unsigned long long*>(take(words * 8));
  w.lpre = static_cast<int32_t*>(take(words * 4));
  w.ncount = static_cast<int32_t*>(take(static_cast<size_t>(g.d_ff) * 4));
  w.offsets = static_cast<int32_t*>(take((static_cast<size_t>(g.d_ff) + 1) * 4));
  // the entries, then (after the weight pass) the dense fallback's partial sums
  const size_t ent_off = off;
  w.ent_row = static_cast<int32_t*>(take(ents * 4));
  w.ent_hz = static_cast<float2*>(take(ents * 8));
  w.part = p == nullptr ? nullptr : reinterpret_cast<float*>(p + ent_off);
  w.part_elems = static_cast<int64_t>((off - ent_off) / 4);
  const size_t sk = skinny_ws_bytes(g);
  w.skinny = static_cast<float*>(take(sk));
  if (sk == 0) w.skinny = nullptr;
  w.bytes = off;
  return w;
}

hipError_t launch_backward(const Geometry& g, int elem_bytes, const BwdHybrid& hy, const void* x,
                           const void* w_up_t, const void* w_down, const void* dy,
                           const BwdWorkspace& w, void* dx, float* dw_up_t, float* db,
                           float* dw_down, hipStream_t s) {
  const int64_t wsize = static_cast<int64_t>(g.d_ff) * g.d_model;
  hipError_t e;
  if (g.n_rows == 0) {  // no rows: every gradient is zero (dx has no rows)
    if ((e = zero_words(dw_up_t, wsize, s)) != hipSuccess) return e;
    if ((e = zero_words(dw_down, wsize, s)) != hipSuccess) return e;
    return zero_words(db, g.d_ff, s);
  }
  const int V = 16 / elem_bytes;
  const int64_t cap = clamp_cap(g, hy.cap);
  const int dchunks = (g.d_ff + kWave * V - 1) / (kWave * V);
  const Items it{g.n_rows, dchunks, g.n_rows + cap * dchunks};
  const unsigned rgrid = grid_for(it.total);
  const int64_t n_words = (g.n_rows + 63) / 64;
  const bool bf = elem_bytes == 2;
  // 1. dz at the non-zeros
  if (bf)
    bwd_dz_kernel<uint16_t><<<rgrid, kBwdThreads, 0, s>>>(
        hy, it, static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(w_down),
        static_cast<uint16_t*>(w.dz_vals), static_cast<uint16_t*>(w.dz_dense), g.d_model, g.d_ff,
        g.tile, g.capacity, g.n_tiles);
  else
    bwd_dz_kernel<float><<<rgrid, kBwdThreads, 0, s>>>(
        hy, it, static_cast<const float*>(dy), static_cast<const float*>(w_down),
        static_cast<float*>(w.dz_vals), static_cast<float*>(w.dz_dense), g.d_model, g.d_ff, g.tile,
        g.capacity, g.n_tiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 2. column lists in row order: bitmap, per-neuron word prefixes, offsets, places
  if ((e = zero_words(w.bits, 2 * n_words * g.d_ff, s)) != hipSuccess) return e;
  auto columns = [&](auto mark) {
    constexpr bool M = decltype(mark)::value;
    if (bf)
      bwd_columns_kernel<uint16_t, M><<<rgrid, kBwdThreads, 0, s>>>(
          hy, it, static_cast<const uint16_t*>(w.dz_vals),
          static_cast<const uint16_t*>(w.dz_dense), g.d_ff, g.tile, g.capacity, g.n_tiles,
          n_words, w.bits, w.lpre, w.offsets, w.ent_row, w.ent_hz);
    else
      bwd_columns_kernel<float, M><<<rgrid, kBwdThreads, 0, s>>>(
          hy, it, static_cast<const float*>(w.dz_vals), static_cast<const float*>(w.dz_dense),
          g.d_ff, g.tile, g.capacity, g.n_tiles, n_words, w.bits, w.lpre, w.offsets, w.ent_row,
          w.ent_hz);
    return hipGetLastError();
  };
  if ((e = columns(std::true_type{})) != hipSuccess) return e;
  bwd_word_prefix_kernel<<<grid_for(g.d_ff), kBwdThreads, 0, s>>>(w.bits, n_words, g.d_ff, w.lpre,
                                                                 w.ncount);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_offsets_kernel<<<1, kBwdScanThreads, 0, s>>>(w.ncount, g.d_ff, w.offsets);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = columns(std::false_type{})) != hipSuccess) return e;
  // 3. weight and bias gradients
  const int n_chunks = (g.d_model + kWave * V - 1) / (kWave * V);
  const int64_t witems = static_cast<int64_t>(g.d_ff) * n_chunks;
  const unsigned wblocks = static_cast<unsigned>((witems + kBwdWaves - 1) / kBwdWaves);
  if (bf)
    bwd_weights_kernel<uint16_t><<<wblocks, kBwdThreads, 0, s>>>(
        w.offsets, w.ent_row, w.ent_hz, static_cast<const uint16_t*>(x),
        static_cast<const uint16_t*>(dy), g.d_ff, g.d_model, n_chunks, dw_up_t, db, dw_down);
  else
    bwd_weights_kernel<float><<<wblocks, kBwdThreads, 0, s>>>(
        w.offsets, w.ent_row, w.ent_hz, static_cast<const float*>(x), static_cast<const float*>(dy),
        g.d_ff, g.d_model, n_chunks, dw_up_t, db, dw_down);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. dx = dz W_up^T: the TwELL rows by the gather kernel, the stored dense
  // rows by the fallback GEMM (its partial sums where the entries were)
  const DenseSkip skip{hy.dense_rows, hy.n_dense, hy.cap};
  if ((e = launch_spmm_sparse(g, elem_bytes, w.dz_vals, hy.idx, hy.cnt, nullptr, nullptr,
                              cap > 0 ? &skip : nullptr, w_up_t, dx, s)) != hipSuccess)
    return e;
  if (cap == 0) return hipSuccess;
  if (bf)
    return launch_fallback_bf16(g, static_cast<const uint16_t*>(w.dz_dense), hy.dense_rows,
                                hy.n_dense, cap, static_cast<const uint16_t*>(w_up_t),
                                static_cast<uint16_t*>(dx), s, w.skinny, w.part, w.part_elems);
  return launch_fallback_f32(g, static_cast<const float*>(w.dz_dense), hy.dense_rows, hy.n_dense,
                             cap, static_cast<const float*>(w_up_t), static_cast<float*>(dx), s,
                             w.skinny);
}

}  // namespace twell
