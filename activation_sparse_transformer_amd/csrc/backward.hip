// The layer's training step: gradients of L = sum(y * dy) from the stored
// hybrid activations ("Sparser, Faster, Lighter Transformer Language Models
// (Sakana AI + NVIDIA)", TL;DR: the format serves training as well as
// inference; "Nvidia and Sakana make LLMs 30% faster by doing less math",
// section "More speed, less power, zero quality loss": faster training with
// lower peak memory).  The ReLU passes gradient exactly where the stored
// activation is non-zero, so every gradient is read from h's non-zeros.
//
// The non-zeros are put in per-neuron lists in ascending row order (a
// (neuron, row) bitmap set with atomic OR, which is order-free, then per-
// neuron prefix counts of its 64-row words give each non-zero's place).  Two
// passes then walk every neuron j's list over column slices of d_model, one
// slice per XCD; per entry (row n, h):
//   A: the slice's partial dot of dy[n] with W_down[j], and
//      dW_down[j] += h * dy[n] over the slice;
//   B: dz = the slices' partial dots added in slice order, rounded to the
//      storage type and written back to the slot it came from (TwELL slot or
//      stored dense element); dW_up^T[j] += dz * x[n] over the slice and
//      db[j] += dz.
// Every sum runs in a fixed order, so every result is a fixed function of the
// input.  dx = dz W_up^T is the hybrid product with dz's values in h's
// slots: the TwELL gather for the sparse rows, the dense fallback GEMM for
// the stored dense rows.
#include <type_traits>

#include "../../include/twell.h"
#include "common.h"
#include "kernels.h"
#include "vec_ops.h"

namespace twell {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdWaves = kBwdThreads / kWave;
constexpr int kBwdScanThreads = 1024;
constexpr int kBwdScanPer = 16;  // elements per thread per round of the offsets scan
constexpr unsigned kBwdMaxBlocks = 65536;

__device__ __forceinline__ int64_t stored_dense(const BwdHybrid& hy) {
  if (hy.cap <= 0) return 0;
  return min(static_cast<int64_t>(max(*hy.n_dense, 0)), hy.cap);
}

// Work items of the row-wise passes: items [0, N) are token rows (their TwELL
// slots; a row flagged as a stored dense row is skipped), items
// N + m * n_chunks + q are column chunk q (64 lanes x 16 bytes) of stored
// dense row m.  Item i is taken by wave i of a grid-stride loop; dense items
// past the stored rows end the loop (they only grow with i).
struct Items {
  int64_t n_rows;
  int n_chunks;
  int64_t total;
};

__device__ __forceinline__ int64_t first_wave() {
  return static_cast<int64_t>(blockIdx.x) * kBwdWaves + threadIdx.x / kWave;
}
__device__ __forceinline__ int64_t wave_stride() {
  return static_cast<int64_t>(gridDim.x) * kBwdWaves;
}

__global__ __launch_bounds__(kBwdThreads) void bwd_zero_kernel(uint32_t* __restrict__ p,
                                                               int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBwdThreads)
    p[i] = 0u;
}

// For each stored dense row m (one wave per (m, chunk) item, items
// m * n_chunks + q below n_items): zero its row of dz_dense and flag its token
// row.  row_flag starts zeroed.
template <typename E>
__global__ __launch_bounds__(kBwdThreads) void bwd_dense_prep_kernel(
    BwdHybrid hy, int64_t n_rows, int64_t n_items, int n_chunks, int dff,
    E* __restrict__ dz_dense, uint8_t* __restrict__ row_flag) {
  constexpr int V = 16 / sizeof(E);
  const int lane = lane_id();
  const int64_t stored = stored_dense(hy);
  for (int64_t i = first_wave(); i < n_items; i += wave_stride()) {
    const int64_t m = i / n_chunks;
    if (m >= stored) break;
    const int q = static_cast<int>(i % n_chunks);
    const int col = q * (kWave * V) + lane * V;
    if (col < dff) *reinterpret_cast<uint4*>(dz_dense + m * dff + col) = make_uint4(0, 0, 0, 0);
    if (q == 0 && lane == 0) {
      const int64_t r = hy.dense_rows[m];
      if (r >= 0 && r < n_rows) row_flag[r] = 1;
    }
  }
}

// Visit every non-zero (neuron j, row n) of h.  MARK sets bit n % 64 of
// bits[j][n / 64]; otherwise the entry {row, h as float32 bits, slot} goes to
// its place offsets[j] + lpre[j][n / 64] + (bits of that word below n % 64).
// slot: n * nt * C + s for TwELL slot s, N * nt * C + m * d_ff + col for the
// stored dense element (m, col).
template <typename E, bool MARK>
__global__ __launch_bounds__(kBwdThreads) void bwd_columns_kernel(
    BwdHybrid hy, Items it, const uint8_t* __restrict__ row_flag, int dff, int T, int C, int nt,
    int64_t n_words, unsigned long long* __restrict__ bits, const int32_t* __restrict__ lpre,
    const int32_t* __restrict__ offsets, int4* __restrict__ ents) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  const int lane = lane_id();
  const int nslots = nt * C;
  const int64_t sparse_slots = it.n_rows * nslots;
  const int64_t stored = stored_dense(hy);
  auto visit = [&](int j, int64_t n, E h, int64_t slot) {
    const int64_t w = static_cast<int64_t>(j) * n_words + (n >> 6);
    const unsigned long long bit = 1ull << (n & 63);
    if constexpr (MARK) {
      atomicOr(bits + w, bit);
    } else {
      const int pos = offsets[j] + lpre[w] + __popcll(bits[w] & (bit - 1));
      ents[pos] = make_int4(static_cast<int>(n), static_cast<int>(__float_as_uint(Tr::to_f32(h))),
                            static_cast<int>(slot), 0);
    }
  };
  for (int64_t i = first_wave(); i < it.total; i += wave_stride()) {
    if (i >= it.n_rows) {
      const int64_t m = (i - it.n_rows) / it.n_chunks;
      if (m >= stored) break;
      const int col = static_cast<int>((i - it.n_rows) % it.n_chunks) * (kWave * V) + lane * V;
      if (col >= dff) continue;
      const int64_t n = hy.dense_rows[m];
      E hv[V];
      *reinterpret_cast<uint4*>(hv) =
          *reinterpret_cast<const uint4*>(static_cast<const E*>(hy.dense_values) + m * dff + col);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (Tr::abs_bits(hv[e]) != 0u) visit(col + e, n, hv[e], sparse_slots + m * dff + col + e);
      continue;
    }
    const int64_t n = i;
    if (row_flag[n]) continue;  // a stored dense row: read from dense_values only
    const E* vrow = static_cast<const E*>(hy.vals) + n * nslots;
    const uint8_t* irow = hy.idx + n * nslots;
    for (int s = lane; s < nslots; s += kWave) {
      const int t = s / C;
      if (s - t * C < static_cast<int>(hy.cnt[n * nt + t])) {
        const int local = irow[s];
        if (local < T) visit(t * T + local, n, vrow[s], n * nslots + s);
      }
    }
  }
}

// Per neuron j (one wave each): lpre[j][b] = set bits of words [0, b) of
// bits[j], and ncount[j] = all its set bits.
__global__ __launch_bounds__(kBwdThreads) void bwd_word_prefix_kernel(
    const unsigned long long* __restrict__ bits, int64_t n_words, int dff,
    int32_t* __restrict__ lpre, int32_t* __restrict__ ncount) {
  const int lane = lane_id();
  const int64_t j = first_wave();
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

// offsets[j] = ncount[0] + ... + ncount[j - 1] for j in [0, dff], one
// workgroup: rounds of kBwdScanThreads * kBwdScanPer elements, thread t
// holding the kBwdScanPer consecutive elements from t * kBwdScanPer (read as
// 16-byte loads; d_ff is a multiple of the tile, so of 4), a wave scan of
// the per-thread totals and one of the wave totals.
__global__ __launch_bounds__(kBwdScanThreads) void bwd_offsets_kernel(
    const int32_t* __restrict__ ncount, int dff, int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[kBwdScanThreads / kWave];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  constexpr int kRound = kBwdScanThreads * kBwdScanPer;
  int carry = 0;
  for (int r0 = 0; r0 < dff; r0 += kRound) {
    const int j0 = r0 + tid * kBwdScanPer;
    int v[kBwdScanPer];
#pragma unroll
    for (int k = 0; k < kBwdScanPer; k += 4) {
      const int4 q = j0 + k < dff ? *reinterpret_cast<const int4*>(ncount + j0 + k)
                                  : make_int4(0, 0, 0, 0);
      v[k] = q.x, v[k + 1] = q.y, v[k + 2] = q.z, v[k + 3] = q.w;
    }
    int local = 0;
#pragma unroll
    for (int k = 0; k < kBwdScanPer; ++k) local += v[k];
    int sc = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(sc, o, kWave);
      if (lane >= o) sc += u;
    }
    if (lane == kWave - 1) wave_tot[wave] = sc;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kBwdScanThreads / kWave; ++w) {
      before += w < wave ? wave_tot[w] : 0;
      total += wave_tot[w];
    }
    int run = carry + before + sc - local;
#pragma unroll
    for (int k = 0; k < kBwdScanPer; ++k) {
      if (j0 + k < dff) offsets[j0 + k] = run;
      run += v[k];
    }
    carry += total;
    __syncthreads();  // wave_tot is rewritten by the next round
  }
  if (tid == 0) offsets[dff] = carry;
}

// The per-neuron passes work on column slices: slice s of S is columns
// [s * sw, (s + 1) * sw) of d_model, and the workgroups of slice s are
// dispatched to the same XCD (block b takes slice b % S, and the hardware
// deals workgroups to its 8 XCDs in turn), so that XCD's L2 holds that slice
// of dy (pass A) or x (pass B) for all of its gathers.  One wave takes one
// neuron j of its block's slice.  It loads j's entry records 64 at a time,
// one per lane; its lanes form 64 / P groups of P lanes, group g taking
// entries g, g + 64 / P, ... of each 64 (their records passed by lane
// shuffles, UP passes of gathers in flight), lane l of a group holding slice
// columns (v * P + l) * V.. for v < NVL.  The groups' sums are added in a
// fixed butterfly order at the end, so every result is a fixed function of
// the input.  part[s * pstride + entry] holds slice s's partial dot of dz.

// A lane's columns of one slice of an fp32 gradient row: acc, or zeros when
// acc is null.
template <int NVL, int V>
__device__ __forceinline__ void write_slice(float* out, const int (&col)[NVL],
                                            const bool (&cok)[NVL], const float* acc) {
#pragma unroll
  for (int v = 0; v < NVL; ++v)
    if (cok[v]) {
#pragma unroll
      for (int i = 0; i < V; i += 4)
        *reinterpret_cast<float4*>(out + col[v] + i) =
            acc == nullptr ? make_float4(0.f, 0.f, 0.f, 0.f)
                           : make_float4(acc[v * V + i], acc[v * V + i + 1], acc[v * V + i + 2],
                                         acc[v * V + i + 3]);
    }
}


// U passes of pass A from entry e0 of the chunk (group g takes entry
// e0 + u * 64 / P + g).  CHECK: some entries may lie past the chunk's cnt;
// their rows are selected away where used (zeroing the load registers
// instead would wait for every load in flight).  Lanes past the slice hold a
// zero W_down and are never written.
template <typename E, int P, int NVL, int U, bool CHECK>
__device__ __forceinline__ void down_step(int e0, int cnt, const int4& mine,
                                          const E* __restrict__ dy, int dm,
                                          const int (&col)[NVL], const uint4 (&wv)[NVL],
                                          float* acc, float& mypd) {
  constexpr int V = 16 / sizeof(E);
  constexpr int GPW = kWave / P;
  const int lane = lane_id(), grp = lane / P;
  uint32_t hb[U];
  uint4 yv[U][NVL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = e0 + u * GPW + grp;
    const int src = CHECK ? min(e, cnt - 1) : e;
    const int row = __shfl(mine.x, src, kWave);
    hb[u] = store_bits<E>(static_cast<uint32_t>(__shfl(mine.y, src, kWave)));
    const int64_t o = static_cast<int64_t>(row) * dm;
#pragma unroll
    for (int v = 0; v < NVL; ++v) yv[u][v] = *reinterpret_cast<const uint4*>(dy + o + col[v]);
  }
  if constexpr (CHECK) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = e0 + u * GPW + grp < cnt;
#pragma unroll
      for (int v = 0; v < NVL; ++v) yv[u][v] = keep_if(live, yv[u][v]);
    }
  }
  float pd[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    pd[u] = 0.f;
#pragma unroll
    for (int v = 0; v < NVL; ++v) pd[u] += dot16<E>(yv[u][v], wv[v]);
  }
  group_totals<P, U>(pd);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // entry e's partial is in the last lane of group e - e_u; lane e takes it
    const int e_u = e0 + u * GPW;
    const float got = __shfl(pd[u], (lane - e_u) * P + P - 1, kWave);
    if (lane >= e_u && lane < e_u + GPW) mypd = got;
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int v = 0; v < NVL; ++v) axpy16<E>(acc + v * V, hb[u], yv[u][v]);
}

// U passes of pass B: dW_up^T += dz * x[n] for the entries from e0.
template <typename E, int P, int NVL, int U, bool CHECK>
__device__ __forceinline__ void up_step(int e0, int cnt, const int4& mine, uint32_t zmine,
                                        const E* __restrict__ x, int dm, const int (&col)[NVL],
                                        float* acc) {
  constexpr int V = 16 / sizeof(E);
  constexpr int GPW = kWave / P;
  const int grp = lane_id() / P;
  uint32_t zb[U];
  uint4 xv[U][NVL];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = e0 + u * GPW + grp;
    const int src = CHECK ? min(e, cnt - 1) : e;
    const int row = __shfl(mine.x, src, kWave);
    zb[u] = static_cast<uint32_t>(__shfl(static_cast<int>(zmine), src, kWave));
    const int64_t o = static_cast<int64_t>(row) * dm;
#pragma unroll
    for (int v = 0; v < NVL; ++v) xv[u][v] = *reinterpret_cast<const uint4*>(x + o + col[v]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool live = !CHECK || e0 + u * GPW + grp < cnt;
#pragma unroll
    for (int v = 0; v < NVL; ++v)
      axpy16<E>(acc + v * V, zb[u], CHECK ? keep_if(live, xv[u][v]) : xv[u][v]);
  }
}

// Pass A: for each entry (row n, h) of neuron j, the partial dot of dy[n]
// with W_down[j] over the slice, stored at part[s * pstride + entry]; and
// dW_down[j][slice] = sum of h * dy[n][slice].
template <typename E, int P, int NVL>
__global__ __launch_bounds__(kBwdThreads) void bwd_slice_down_kernel(
    const int32_t* __restrict__ offsets, const int4* __restrict__ ents, const E* __restrict__ dy,
    const E* __restrict__ w_down, int dff, int dm, int S, int sw, float* __restrict__ part,
    int64_t pstride, float* __restrict__ dw_down) {
  constexpr int V = 16 / sizeof(E);
  constexpr int GPW = kWave / P;                              // entries per pass
  constexpr int UP = GPW * NVL >= 8 ? 1 : 8 / (GPW * NVL);  // passes in flight
  const int lane = lane_id(), grp = lane / P, l = lane % P;
  const int s = blockIdx.x % S;
  const int j = (blockIdx.x / S) * kBwdWaves + threadIdx.x / kWave;
  if (j >= dff) return;
  const int cs = s * sw;
  int col[NVL];
  bool cok[NVL];
#pragma unroll
  for (int v = 0; v < NVL; ++v) {
    const int c = (v * P + l) * V;
    cok[v] = c < sw;
    col[v] = cs + (cok[v] ? c : 0);  // a lane past the slice reads its first column, zeroed
  }
  float* out = dw_down + static_cast<int64_t>(j) * dm;
  const int b = offsets[j], L = offsets[j + 1] - b;
  if (L == 0) {  // no entry: a zero row, W_down[j] not read
    if (grp == 0) write_slice<NVL, V>(out, col, cok, nullptr);
    return;
  }
  const E* wrow = w_down + static_cast<int64_t>(j) * dm;
  uint4 wv[NVL];
#pragma unroll
  for (int v = 0; v < NVL; ++v)
    wv[v] = cok[v] ? *reinterpret_cast<const uint4*>(wrow + col[v]) : make_uint4(0, 0, 0, 0);
  float acc[NVL * V];
#pragma unroll
  for (int i = 0; i < NVL * V; ++i) acc[i] = 0.f;
  for (int base = 0; base < L; base += kWave) {
    const int cnt = min(kWave, L - base);
    const int4 mine = ents[b + base + min(lane, cnt - 1)];
    float mypd = 0.f;  // lane t: the partial dot of the chunk's entry t
    int e0 = 0;
    for (; e0 + GPW * UP <= cnt; e0 += GPW * UP)
      down_step<E, P, NVL, UP, false>(e0, cnt, mine, dy, dm, col, wv, acc, mypd);
    for (; e0 < cnt; e0 += GPW)
      down_step<E, P, NVL, 1, true>(e0, cnt, mine, dy, dm, col, wv, acc, mypd);
    // slice-major: the chunk's partials are one coalesced store
    if (lane < cnt) part[s * pstride + b + base + lane] = mypd;
  }
#pragma unroll
  for (int o = P; o < kWave; o <<= 1)
#pragma unroll
    for (int i = 0; i < NVL * V; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
  if (grp == 0) write_slice<NVL, V>(out, col, cok, acc);
}

// Pass B: per entry dz = the S partial dots added in slice order, rounded to
// E (each lane finishes the dz of its own entry record; slice 0 stores it at
// the entry's slot and adds it to db[j]); and dW_up^T[j][slice] = sum of
// dz * x[n][slice].
template <typename E, int P, int NVL>
__global__ __launch_bounds__(kBwdThreads) void bwd_slice_up_kernel(
    const int32_t* __restrict__ offsets, const int4* __restrict__ ents, const E* __restrict__ x,
    const float* __restrict__ part, int64_t pstride, int dff, int dm, int S, int sw,
    int64_t sparse_slots,
    E* __restrict__ dz_vals, E* __restrict__ dz_dense, float* __restrict__ dw_up_t,
    float* __restrict__ db) {
  typedef ElemTraits<E> Tr;
  constexpr int V = 16 / sizeof(E);
  constexpr int GPW = kWave / P;
  constexpr int UP = GPW * NVL >= 8 ? 1 : 8 / (GPW * NVL);
  const int lane = lane_id(), grp = lane / P, l = lane % P;
  const int s = blockIdx.x % S;
  const int j = (blockIdx.x / S) * kBwdWaves + threadIdx.x / kWave;
  if (j >= dff) return;
  const int cs = s * sw;
  int col[NVL];
  bool cok[NVL];
#pragma unroll
  for (int v = 0; v < NVL; ++v) {
    const int c = (v * P + l) * V;
    cok[v] = c < sw;
    col[v] = cs + (cok[v] ? c : 0);
  }
  const int b = offsets[j], L = offsets[j + 1] - b;
  if (L == 0) {  // no entry: zero rows and bias
    if (grp == 0) write_slice<NVL, V>(dw_up_t + static_cast<int64_t>(j) * dm, col, cok, nullptr);
    if (s == 0 && lane == 0) db[j] = 0.f;
    return;
  }
  float acc[NVL * V];
#pragma unroll
  for (int i = 0; i < NVL * V; ++i) acc[i] = 0.f;
  float sdz = 0.f;  // slice 0: lane l's entries' dz, added over the chunks
  for (int base = 0; base < L; base += kWave) {
    const int cnt = min(kWave, L - base);
    const int64_t me = b + base + min(lane, cnt - 1);
    const int4 mine = ents[me];
    float d;
    if (S == 8) {  // the 8 partials, each load coalesced over the lanes, added in slice order
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) p[t] = part[t * pstride + me];
      d = ((((((p[0] + p[1]) + p[2]) + p[3]) + p[4]) + p[5]) + p[6]) + p[7];
    } else {
      d = part[me];
      for (int t = 1; t < S; ++t) d += part[t * pstride + me];
    }
    const E dze = Tr::from_f32(d);
    const float dzf = lane < cnt ? Tr::to_f32(dze) : 0.f;
    const uint32_t zmine = store_bits<E>(__float_as_uint(dzf));
    int e0 = 0;
    for (; e0 + GPW * UP <= cnt; e0 += GPW * UP)
      up_step<E, P, NVL, UP, false>(e0, cnt, mine, zmine, x, dm, col, acc);
    for (; e0 < cnt; e0 += GPW) up_step<E, P, NVL, 1, true>(e0, cnt, mine, zmine, x, dm, col, acc);
    // after the gathers, so the loop above never waits for these stores
    if (s == 0 && lane < cnt) {
      const int64_t slot = mine.z;
      if (slot < sparse_slots) dz_vals[slot] = dze;
      else dz_dense[slot - sparse_slots] = dze;
      sdz += dzf;
    }
  }
#pragma unroll
  for (int o = P; o < kWave; o <<= 1)
#pragma unroll
    for (int i = 0; i < NVL * V; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
  if (grp == 0) write_slice<NVL, V>(dw_up_t + static_cast<int64_t>(j) * dm, col, cok, acc);
  if (s == 0) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) sdz += __shfl_xor(sdz, o, kWave);
    if (lane == 0) db[j] = sdz;
  }
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

// Column slices of the per-neuron passes: 8 (one per XCD) when d_model splits
// into 8 whole 16-byte groups, else 1; P lanes and nvl vectors per lane cover
// one slice's sw columns (nvl = 0: the slice is too wide).
SlicePlan bwd_slice_plan(int d_model, int elem_bytes) {
  const int V = 16 / elem_bytes;
  SlicePlan p;
  p.S = d_model % (8 * V) == 0 ? 8 : 1;
  p.sw = d_model / p.S;
  const int vs = (p.sw + V - 1) / V;
  p.P = vs <= 8 ? 8 : vs <= 16 ? 16 : vs <= 32 ? 32 : kWave;
  const int nvl = (vs + p.P - 1) / p.P;
  p.nvl = nvl <= 1 ? 1 : nvl <= 2 ? 2 : nvl <= 4 ? 4 : 0;
  return p;
}

namespace {

template <typename E, int P, int NVL>
hipError_t launch_slices(const Geometry& g, const SlicePlan& sp, const BwdWorkspace& w,
                         const void* x, const void* dy, const void* w_down, float* dw_up_t,
                         float* db, float* dw_down, hipStream_t s) {
  const unsigned blocks =
      static_cast<unsigned>((g.d_ff + kBwdWaves - 1) / kBwdWaves) * static_cast<unsigned>(sp.S);
  bwd_slice_down_kernel<E, P, NVL><<<blocks, kBwdThreads, 0, s>>>(
      w.offsets, w.ents, static_cast<const E*>(dy), static_cast<const E*>(w_down), g.d_ff,
      g.d_model, sp.S, sp.sw, w.part_dz, w.part_stride, dw_down);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_slice_up_kernel<E, P, NVL><<<blocks, kBwdThreads, 0, s>>>(
      w.offsets, w.ents, static_cast<const E*>(x), w.part_dz, w.part_stride, g.d_ff, g.d_model,
      sp.S, sp.sw,
      g.n_rows * g.n_tiles * g.capacity, static_cast<E*>(w.dz_vals),
      static_cast<E*>(w.dz_dense), dw_up_t, db);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_neuron_pass(const Geometry& g, const BwdWorkspace& w, const void* x,
                              const void* dy, const void* w_down, float* dw_up_t, float* db,
                              float* dw_down, hipStream_t s) {
  const SlicePlan sp = bwd_slice_plan(g.d_model, sizeof(E));
  switch (sp.P * 8 + sp.nvl) {
    case 8 * 8 + 1: return launch_slices<E, 8, 1>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    case 16 * 8 + 1: return launch_slices<E, 16, 1>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    case 32 * 8 + 1: return launch_slices<E, 32, 1>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    case 64 * 8 + 1: return launch_slices<E, 64, 1>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    case 64 * 8 + 2: return launch_slices<E, 64, 2>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    case 64 * 8 + 4: return launch_slices<E, 64, 4>(g, sp, w, x, dy, w_down, dw_up_t, db, dw_down, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool bwd_supported(const Geometry& g, int elem_bytes) {
  return bwd_slice_plan(g.d_model, elem_bytes).nvl != 0;
}

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
  // bits and row flags are one zeroed region
  const size_t zero_off = off;
  w.bits = static_cast<unsigned long long*>(take(words * 8));
  w.row_flag = static_cast<uint8_t*>(take(static_cast<size_t>(g.n_rows)));
  w.zero_words = static_cast<int64_t>((off - zero_off) / 4);
  w.dz_vals = take(slots * elem_bytes);
  w.dz_dense = take(cap * g.d_ff * elem_bytes);
  w.lpre = static_cast<int32_t*>(take(words * 4));
  w.ncount = static_cast<int32_t*>(take(static_cast<size_t>(g.d_ff) * 4));
  w.offsets = static_cast<int32_t*>(take((static_cast<size_t>(g.d_ff) + 1) * 4));
  // the entries and the slices' partial dots, then (after the per-neuron
  // passes) the dense fallback's partial sums
  const size_t ent_off = off;
  w.ents = static_cast<int4*>(take(ents * sizeof(int4)));
  const SlicePlan sp = bwd_slice_plan(g.d_model, elem_bytes);
  w.part_dz = static_cast<float*>(take(static_cast<size_t>(sp.S) * ents * sizeof(float)));
  w.part_stride = static_cast<int64_t>(ents);
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
  // 1. clear the bitmap and row flags; zero the stored dense rows' dz, flag their rows
  if ((e = zero_words(w.bits, w.zero_words, s)) != hipSuccess) return e;
  if (cap > 0) {
    const int64_t items = cap * dchunks;
    const unsigned dgrid = grid_for(items);
    if (bf)
      bwd_dense_prep_kernel<uint16_t><<<dgrid, kBwdThreads, 0, s>>>(
          hy, g.n_rows, items, dchunks, g.d_ff, static_cast<uint16_t*>(w.dz_dense), w.row_flag);
    else
      bwd_dense_prep_kernel<float><<<dgrid, kBwdThreads, 0, s>>>(
          hy, g.n_rows, items, dchunks, g.d_ff, static_cast<float*>(w.dz_dense), w.row_flag);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 2. per-neuron lists in row order: bitmap, per-neuron word prefixes, offsets, places
  auto columns = [&](auto mark) {
    constexpr bool M = decltype(mark)::value;
    if (bf)
      bwd_columns_kernel<uint16_t, M><<<rgrid, kBwdThreads, 0, s>>>(
          hy, it, w.row_flag, g.d_ff, g.tile, g.capacity, g.n_tiles, n_words, w.bits, w.lpre,
          w.offsets, w.ents);
    else
      bwd_columns_kernel<float, M><<<rgrid, kBwdThreads, 0, s>>>(
          hy, it, w.row_flag, g.d_ff, g.tile, g.capacity, g.n_tiles, n_words, w.bits, w.lpre,
          w.offsets, w.ents);
    return hipGetLastError();
  };
  if ((e = columns(std::true_type{})) != hipSuccess) return e;
  bwd_word_prefix_kernel<<<grid_for(g.d_ff), kBwdThreads, 0, s>>>(w.bits, n_words, g.d_ff, w.lpre,
                                                                 w.ncount);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_offsets_kernel<<<1, kBwdScanThreads, 0, s>>>(w.ncount, g.d_ff, w.offsets);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = columns(std::false_type{})) != hipSuccess) return e;
  // 3. dz at every entry, weight and bias gradients (two passes over column slices)
  e = bf ? launch_neuron_pass<uint16_t>(g, w, x, dy, w_down, dw_up_t, db, dw_down, s)
         : launch_neuron_pass<float>(g, w, x, dy, w_down, dw_up_t, db, dw_down, s);
  if (e != hipSuccess) return e;
  // 4. dx = dz W_up^T: every row by the TwELL gather (a stored dense row has
  // no live slot, so it gets 0 there), then the stored dense rows by the
  // fallback GEMM over dz_dense (its partial sums where the entries were)
  if ((e = launch_spmm_sparse(g, elem_bytes, w.dz_vals, hy.idx, hy.cnt, nullptr, nullptr, nullptr,
                              w_up_t, dx, s)) != hipSuccess)
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
