// Host-side launchers of the TwELL kernels (internal to libtwell.so).
// Every launcher only enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

// Output side of the TwELL pack step shared by the fused up-projection and
// the standalone dense_to_twell.
struct PackOut {
  void* vals;        // [N][nt][C] dtype
  uint8_t* idx;      // [N][nt][C]
  uint8_t* cnt;      // [N][nt]
  uint8_t* flags;    // [N][nt] workspace: 1 when the tile overflowed
  void* spill;       // [N][d_ff] workspace or nullptr: raw h of overflowing tiles
  void* h_debug;     // [N][d_ff] or nullptr: every h element as packed
  float* skinny;     // skinny_ws_bytes(g) of workspace, or nullptr
};

struct Geometry {
  int64_t n_rows;
  int d_model;
  int d_ff;
  int tile;
  int capacity;
  int n_tiles;
};

// Batches of at most kSkinnyMaxRows rows take split-K "skinny" kernels for
// the up-projection and the fallback when the caller passes skinny_ws_bytes(g)
// of workspace (0 for larger batches): workgroup (column block, slice) writes
// fp32 partial sums part[slice][m][n] (row stride mm), and a second kernel adds
// the slices in slice order and applies the epilogue.
constexpr int64_t kSkinnyMaxRows = 64;
constexpr int kSkinnyMaxSlices = 32;
struct SkinnySplit {
  int slices;  // K slices (<= kSkinnyMaxSlices)
  int kw;      // K per slice, a multiple of the kernel's granule; the last may be shorter
  int mm;      // rows per slice block of the partials: 16, 32 or 64
};
// Enough slices for about target_blocks workgroups over n_blocks column blocks.
SkinnySplit skinny_split(int64_t n_rows, int K, int n_blocks, int granule, int target_blocks);
size_t skinny_ws_bytes(const Geometry& g);
// fp32 inputs: VALU partial kernels.
hipError_t launch_skinny_up_pack_f32(const Geometry& g, const float* x, const float* w_up_t,
                                     const float* b_up, const PackOut& out, float* part,
                                     hipStream_t s);
hipError_t launch_skinny_fallback_f32(const Geometry& g, const float* a, const int32_t* dense_rows,
                                      const int32_t* n_dense, int64_t dense_cap,
                                      const float* w_down, float* y, float* part, hipStream_t s);
// Second halves, shared with the bf16 MFMA partial kernels.
template <typename E>
hipError_t launch_skinny_up_epilogue(const Geometry& g, const SkinnySplit& sp, const float* part,
                                     const float* b_up, const PackOut& out, hipStream_t s);
template <typename E>
hipError_t launch_skinny_fallback_reduce(const Geometry& g, const SkinnySplit& sp,
                                         const float* part, const int32_t* n_dense, int m_cap,
                                         const int32_t* dense_rows, E* y, hipStream_t s);

// G1: h = ReLU(x w_up_t^T + b) rounded to dtype, packed per (row, tile).
hipError_t launch_up_pack_bf16(const Geometry& g, const uint16_t* x, const uint16_t* w_up_t,
                               const float* b_up, const PackOut& out, hipStream_t s);
hipError_t launch_up_pack_f32(const Geometry& g, const float* x, const float* w_up_t,
                              const float* b_up, const PackOut& out, hipStream_t s);

// G5 first half: pack an existing h [N][d_ff] per (row, tile).
hipError_t launch_pack_tiles(const Geometry& g, const void* h, int elem_bytes, const PackOut& out,
                             hipStream_t s);

// Routing scratch (workspace).
struct RouteBufs {
  uint8_t* flags;        // [N][nt] 1 when the tile overflowed (written by the pack step)
  uint8_t* row_dense;    // [N] 1 when any tile of the row overflowed
  int32_t* row_map;      // [N] dense index m of a dense row, -1 for a sparse row
  int32_t* sparse_rows;  // [N] the sparse rows, ascending
  int32_t* n_sparse;     // [1]
};

// G2a: per-row OR of the tile flags, then an ascending numbering of the dense
// rows (one workgroup, block prefix scan):  row_map, dense_rows[m] = n for
// m < dense_cap, *n_dense = total, sparse_rows / *n_sparse, and *status =
// OK / DENSE_CAPACITY.
hipError_t launch_route_scan(const Geometry& g, const RouteBufs& rb, int32_t* dense_rows,
                             int64_t dense_cap, int32_t* n_dense, int32_t* status, hipStream_t s);

// G2b: dense_values[m] = row n of h (from `full_src` if given, else from the
// TwELL slots of the row plus the spilled overflowing tiles), then the row's
// TwELL slots are cleared.
// Routing outputs written by a dense-row build that routes the rows itself;
// row_dense (one 0/1 byte per row) is given when the build counts the dense
// rows below each row from it, and null when each workgroup ORs the tile flags
// of all rows itself (at most 64 rows).
struct RouteOut {
  int64_t n_rows;
  int32_t* dense_rows;
  int32_t* n_dense;
  int32_t* sparse_rows;
  int32_t* n_sparse;
  int32_t* status;
  const uint8_t* row_dense;
  const int32_t* blk_cnt = nullptr;  // dense rows per block of row_or_kernel's rows
};

// The down-projection operands of a dense-row build that also runs the
// sparse product of the sparse rows (float32, at most 64 rows).
struct BuildSpmm {
  const void* w_down;
  void* y;
};

// Whether launch_route_materialize can take a BuildSpmm for this shape: float32,
// the rows routed inside the build (route_mode 1), rows built in LDS, and a
// shape for which launch_spmm_sparse would run the 16-range few-row kernel, so
// that y is the same bits either way.
bool build_takes_spmm(const Geometry& g, int elem_bytes);

hipError_t launch_materialize(const Geometry& g, int elem_bytes, const int32_t* row_map,
                              const uint8_t* flags, const void* spill, const void* full_src,
                              void* vals, uint8_t* idx, uint8_t* cnt, void* dense_values,
                              int64_t dense_cap, hipStream_t s, const RouteOut* route = nullptr,
                              const BuildSpmm* sp = nullptr);

// G2 without the scan kernel: route_mode says whether the dense-row build can
// route the rows itself (1: at most 64 rows, each workgroup ORs every row's
// tile flags and numbers the dense rows with one ballot; 2: more than 1024
// and at most 16384 rows, row_or_kernel first, then the build numbers the
// dense rows from row_dense and the per-block dense counts) or not (0).  Writes what
// launch_route_scan and launch_materialize write, except row_map (and, in mode
// 1, row_dense).  full_src: h when the rows are copied from it (twell_pack).
int route_mode(const Geometry& g);
hipError_t launch_route_materialize(const Geometry& g, int elem_bytes, const RouteBufs& rb,
                                    const void* spill, const void* full_src, void* vals,
                                    uint8_t* idx, uint8_t* cnt, int32_t* dense_rows,
                                    void* dense_values, int64_t dense_cap, int32_t* n_dense,
                                    int32_t* status, hipStream_t s,
                                    const BuildSpmm* sp = nullptr);

// G6: twell_to_dense.
hipError_t launch_unpack(const Geometry& g, int elem_bytes, const void* vals, const uint8_t* idx,
                         const uint8_t* cnt, const int32_t* dense_rows, const void* dense_values,
                         const int32_t* n_dense, int64_t dense_cap, void* h, hipStream_t s);

// Rows the sparse product leaves alone when it walks every row: the stored
// dense rows dense_rows[0 .. min(*n_dense, cap)), ascending (cap 0: none).
struct DenseSkip {
  const int32_t* dense_rows;
  const int32_t* n_dense;
  int64_t cap;
};

// G3: y[n] = sum of value * w_down[row] over the stored slots of row n, for
// the rows rows[0 .. *n_rows_dev) when `rows` is given, else for every row
// that `skip` (may be null) does not list.
hipError_t launch_spmm_sparse(const Geometry& g, int elem_bytes, const void* vals,
                              const uint8_t* idx, const uint8_t* cnt, const int32_t* rows,
                              const int32_t* n_rows_dev, const DenseSkip* skip,
                              const void* w_down, void* y, hipStream_t s);

// G4: y[dense_rows[m]] = dense_values[m] w_down for m < min(*n_dense, dense_cap).
// `skinny`: skinny_ws_bytes(g) of workspace for the split-K path, or nullptr.
// `part`: part_elems floats of scratch in which the 128 x 128 tile kernel may
// keep the partial sums of a K split when few rows are live, or nullptr.
hipError_t launch_fallback_bf16(const Geometry& g, const uint16_t* dense_values,
                                const int32_t* dense_rows, const int32_t* n_dense,
                                int64_t dense_cap, const uint16_t* w_down, uint16_t* y,
                                hipStream_t s, float* skinny = nullptr, float* part = nullptr,
                                int64_t part_elems = 0);

// The few-row sparse product's launch plan for workgroups of `waves` waves,
// each taking `parts_per_wave` of the row's waves * parts_per_wave tile
// ranges: column slices, columns per lane, tiles per range, workgroups, LDS
// bytes.  False when launch_spmm_sparse would not take that kernel.
struct SpmmSplitPlan {
  int n_slices, vec, tpw;
  unsigned blocks;
  size_t lds_bytes;
};
bool spmm_split_plan(const Geometry& g, int waves, int parts_per_wave, SpmmSplitPlan* plan);

// The TwELL rows the sparse product reads (bf16 values).
struct SpmmRows {
  const uint16_t* vals;
  const uint8_t* idx;
  const uint8_t* cnt;
  const int32_t* rows;    // the sparse rows, ascending
  const int32_t* n_rows;  // device count of rows
};

// Batches of at most 64 rows (bf16): whether launch_fallback_bf16_with_spmm
// can run the sparse product inside the fallback's split-K partial-sum launch
// (extra workgroups of the same size, their slot lists in its LDS), and that
// launch: y of the sparse rows, then the fallback's slice sums for the dense
// rows, as launch_spmm_sparse followed by launch_fallback_bf16.
bool fallback_takes_spmm(const Geometry& g);
hipError_t launch_fallback_bf16_with_spmm(const Geometry& g, const uint16_t* dense_values,
                                          const int32_t* dense_rows, const int32_t* n_dense,
                                          int64_t dense_cap, const uint16_t* w_down, uint16_t* y,
                                          hipStream_t s, float* skinny, const SpmmRows& sr);
hipError_t launch_fallback_f32(const Geometry& g, const float* dense_values,
                               const int32_t* dense_rows, const int32_t* n_dense,
                               int64_t dense_cap, const float* w_down, float* y, hipStream_t s,
                               float* skinny = nullptr);

// ELL rows (one tile spanning the row, 16-bit columns; g.capacity = width W).
// Pack: counts, routing (rb.flags holds one flag per row), slots / dense rows.
hipError_t launch_ell_pack(const Geometry& g, int elem_bytes, const void* h, const RouteBufs& rb,
                           void* vals, uint16_t* cols, uint16_t* cnt, int32_t* dense_rows,
                           void* dense_values, int64_t dense_cap, int32_t* n_dense,
                           int32_t* status, hipStream_t s);
// LDS bytes the unpack kernel needs (one row of h).
size_t ell_unpack_lds_bytes(const Geometry& g, int elem_bytes);
hipError_t launch_ell_unpack(const Geometry& g, int elem_bytes, const void* vals,
                             const uint16_t* cols, const uint16_t* cnt, const int32_t* dense_rows,
                             const void* dense_values, const int32_t* n_dense, int64_t dense_cap,
                             void* h, hipStream_t s);
// y of every row that `skip` does not list, from its slots.
hipError_t launch_ell_spmm_sparse(const Geometry& g, int elem_bytes, const void* vals,
                                  const uint16_t* cols, const uint16_t* cnt, const DenseSkip& skip,
                                  const void* w_down, void* y, hipStream_t s);

// The layer's backward pass from the stored hybrid h (dz at h's non-zeros,
// per-neuron weight and bias sums in row order, dx by the hybrid product).
struct BwdHybrid {
  const void* vals;
  const uint8_t* idx;
  const uint8_t* cnt;
  const int32_t* dense_rows;
  const void* dense_values;
  const int32_t* n_dense;
  int64_t cap;
};
struct BwdWorkspace {
  unsigned long long* bits;     // [d_ff][ceil(N / 64)] (neuron, row) bitmap
  uint8_t* row_flag;            // [N] 1 for a stored dense row
  int64_t zero_words;           // 4-byte words of bits + row_flag, cleared together
  void* dz_vals;                // [N][nt][C] dtype
  void* dz_dense;               // [min(cap, N)][d_ff] dtype
  int32_t* lpre;                // [d_ff][ceil(N / 64)] set bits before each word
  int32_t* ncount;              // [d_ff] entries per neuron
  int32_t* offsets;             // [d_ff + 1] first entry of each neuron
  int4* ents;                   // [entries] {row, h as f32 bits, slot, 0}, by neuron then row
  float* part_dz;               // [S][part_stride] partial dots of dz per column slice
  int64_t part_stride;          // entries per slice of part_dz
  float* part;                  // the entry area, reused for the fallback's partial sums
  int64_t part_elems;
  float* skinny;                // skinny_ws_bytes(g) or nullptr
  size_t bytes;                 // total workspace bytes
};
// Column slices of the backward's per-neuron passes: S slices of sw columns,
// P lanes and nvl 16-byte vectors per lane per slice (nvl = 0: unsupported).
struct SlicePlan {
  int S, sw, P, nvl;
};
SlicePlan bwd_slice_plan(int d_model, int elem_bytes);
// Whether the backward covers this d_model (a slice of at most 64 lanes x 4
// vectors x 16 bytes: 16384 bf16 or 8192 fp32 columns when d_model splits in
// 8 slices, 2048 / 1024 otherwise).
bool bwd_supported(const Geometry& g, int elem_bytes);
// Entries the column lists may hold: every TwELL slot and every element of
// the stored dense rows.
int64_t bwd_max_entries(const Geometry& g, int64_t dense_cap);
// Parts of a workspace at `ws` (nullptr: sizes only, in .bytes).
BwdWorkspace bwd_carve(const Geometry& g, int elem_bytes, int64_t dense_cap, void* ws);
hipError_t launch_backward(const Geometry& g, int elem_bytes, const BwdHybrid& hy, const void* x,
                           const void* w_up_t, const void* w_down, const void* dy,
                           const BwdWorkspace& w, void* dx, float* dw_up_t, float* db,
                           float* dw_down, hipStream_t s);

// The ReLU-gated FFN's up branch on a packed and routed gate: each stored
// non-zero g (TwELL slots of the sparse rows sparse_rows[0 .. *n_sparse),
// non-zeros of the stored dense rows) becomes g * (x[n] . w_up_t[j] + b_up[j])
// rounded to the storage type, in place.
struct GateHybrid {
  void* vals;
  const uint8_t* idx;
  const uint8_t* cnt;
  const int32_t* dense_rows;
  void* dense_values;
  const int32_t* n_dense;
  int64_t cap;
  const int32_t* sparse_rows;
  const int32_t* n_sparse;
};
// Whether launch_gate_up covers this shape (d_model up to 16 x 64 x 16 bytes).
bool gate_supported(const Geometry& g, int elem_bytes);
hipError_t launch_gate_up(const Geometry& g, int elem_bytes, const GateHybrid& hy, const void* x,
                          const void* w_up_t, const float* b_up, hipStream_t s);

}  // namespace twell
