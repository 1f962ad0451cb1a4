/*
 * twell.h - C ABI of libtwell.so: the forward pass of a ReLU-activation-sparse
 * transformer feed-forward layer whose hidden activations are stored in the
 * hybrid Tile-wise ELLPACK (TwELL) format, on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on "Sparser, Faster, Lighter Transformer Language Models",
 * Sakana AI + NVIDIA):
 *  - "Sparser, Faster, Lighter Transformer Language Models (Sakana AI +
 *    NVIDIA)" (wiki note), Figure 1 description and packing-format flowchart:
 *    TwELL keeps, per column tile of width T (tile index t), a values array of
 *    the non-zeros only, their tile-local indices and a per-tile non-zero
 *    count; the hybrid variant splits token rows between TwELL and a dense
 *    matrix according to how their non-zeros distribute.
 *  - "Nvidia and Sakana make LLMs 30% faster by doing less math", section
 *    "Reshaping math for the GPU": sparse tokens take the fast path, the rare
 *    dense tokens go to a dense matrix ("safety valve").
 *  - "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse Transformers Run
 *    Like They Were Built for Hopper", section "TwELL: The Packing Format That
 *    Fits the Machine": dense-to-TwELL, TwELL-to-dense and fused MLP execution.
 *  - "The Relentless Search for Efficiency in Large-Scale Language Models",
 *    section "The Challenge of Sparsity Ignored by GPUs": a hidden unit is
 *    active when it is non-zero after the ReLU.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers on the current HIP device,
 *    16-byte aligned, owned by the caller.  The library never allocates or
 *    frees memory and keeps no state between calls (twell_pack_noalloc's
 *    fixed device scratch array is the one exception, by design).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; nothing is
 *    synchronised on the host.  Outputs are valid once the stream reaches the
 *    enqueued work.  Calls are thread-safe; calls that share output or
 *    workspace buffers must be ordered by the caller.
 *  - Return value: TWELL_OK (0) or a negative twell_status.  Argument errors
 *    are detected on the host before anything is enqueued.  Conditions only
 *    known on the device are reported through the optional device word
 *    `d_status` (see TWELL_ERR_DENSE_CAPACITY).
 *  - Element type: `dtype` = TWELL_F32 (IEEE float) or TWELL_BF16 (bfloat16
 *    bits).  x, the weights, y, TwELL values and dense rows all use it; the
 *    up-projection bias is always float32; accumulation is always float32;
 *    results are rounded to the storage type round-to-nearest-even.
 *
 * Layouts (row-major, C order; nt = d_ff / tile)
 *  - x       [n_rows][d_model]
 *  - w_up_t  [d_ff][d_model]  W_up stored transposed (one row per neuron)
 *  - b_up    [d_ff] float32
 *  - w_down  [d_ff][d_model]  one row of W_down per neuron
 *  - y, h    [n_rows][d_model] / [n_rows][d_ff]
 *  - TwELL   values [n_rows][nt][capacity], indices [n_rows][nt][capacity]
 *            uint8, counts [n_rows][nt] uint8
 *
 * Format rules (readings of the pages where they are silent)
 *  - Tile t of a row is columns [t*tile, (t+1)*tile).  Inside a tile the
 *    non-zeros are kept in ascending column order; slot k holds the k-th.
 *  - A value is non-zero when it is != 0 in the storage type (-0.0 is zero,
 *    NaN is non-zero).  The ReLU writes +0.0 for inactive units.
 *  - A tile overflows when its count exceeds `capacity`.  One overflowing
 *    tile makes the whole token row dense: its counts are 0, all its slots
 *    are padding, and its full row is stored in dense_values.  Dense rows are
 *    listed in ascending token order.
 *  - Padding slots hold value +0.0 (all-zero bits) and index 0.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWELL_VERSION 1

typedef enum twell_status {
  TWELL_OK = 0,
  TWELL_ERR_INVALID_ARG = -1,    /* null pointer, negative size, bad geometry */
  TWELL_ERR_UNSUPPORTED = -2,    /* valid TwELL geometry the library has no kernel for */
  TWELL_ERR_WORKSPACE = -3,      /* workspace smaller than the *_workspace_size query */
  TWELL_ERR_HIP = -4,            /* a HIP launch failed */
  TWELL_ERR_DENSE_CAPACITY = -5, /* device-side: more dense rows than dense_capacity */
  TWELL_ERR_SCRATCH_LIMIT = -6   /* the shape needs more than the fixed device scratch */
} twell_status;

typedef enum twell_dtype { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype;

/* Shape of one FFN layer and its TwELL geometry (tile width T and capacity
 * C of "Sparser, Faster, Lighter Transformer Language Models (Sakana AI +
 * NVIDIA)", Figure 1 description; the configuration names T and C, the pages
 * name T and the tile index t).
 * Requirements: n_rows >= 0 and < 2^31; d_model > 0 and a multiple of 8;
 * d_ff > 0 and a multiple of tile; tile in {64, 128, 256} (other tile widths
 * are TWELL_ERR_UNSUPPORTED); 1 <= capacity <= min(tile, 255); dtype a
 * twell_dtype.  d_model is ignored by twell_pack and twell_unpack. */
typedef struct twell_shape {
  int64_t n_rows;   /* N, tokens */
  int32_t d_model;  /* model width */
  int32_t d_ff;     /* hidden width */
  int32_t tile;     /* T, tile width */
  int32_t capacity; /* C, slots per tile */
  int32_t dtype;    /* twell_dtype */
  int32_t reserved; /* must be 0 */
} twell_shape;

/* A hybrid TwELL matrix [n_rows][d_ff] (all device pointers, caller-owned):
 * the values / tile-local indices / per-tile counts of "Sparser, Faster,
 * Lighter Transformer Language Models (Sakana AI + NVIDIA)", Figure 1
 * description (panel b), plus the dense rows of its hybrid split (panel c).
 *  values       [n_rows][nt][capacity]   dtype
 *  indices      [n_rows][nt][capacity]   uint8, tile-local column
 *  counts       [n_rows][nt]             uint8
 *  dense_rows   [dense_capacity]         int32, ascending token rows
 *  dense_values [dense_capacity][d_ff]   dtype, the dense rows bit for bit
 *  n_dense      device int32: number of dense rows (may exceed
 *               dense_capacity after a TWELL_ERR_DENSE_CAPACITY pack; only
 *               the first dense_capacity are stored)
 * dense_rows / dense_values may be NULL when dense_capacity == 0. */
typedef struct twell_hybrid {
  void* values;
  uint8_t* indices;
  uint8_t* counts;
  int32_t* dense_rows;
  void* dense_values;
  int32_t* n_dense;
  int64_t dense_capacity;
} twell_hybrid;

/* Library version (TWELL_VERSION).  Defined by this interface, not by the
 * pages. */
int twell_version(void);

/* Static string naming a twell_status value ("unknown status" otherwise).
 * Defined by this interface, not by the pages. */
const char* twell_status_string(int status);

/* Bytes of device workspace ffn_sparse_forward needs for this shape
 * (0 for an invalid shape).  Sized for the worst case: every tile spilled;
 * batches of at most 64 rows add room for fp32 split-K partial sums.
 * The scratch behind the fused pass of "SakanaAI/sparser-faster-llms: How
 * TwELL Makes Sparse Transformers Run Like They Were Built for Hopper",
 * section "TwELL: The Packing Format That Fits the Machine". */
size_t ffn_sparse_workspace_size(const twell_shape* shape);

/* The fused forward pass: y = ReLU(x W_up + b_up) W_down, with the hidden
 * activations h produced directly in hybrid TwELL form.
 * Defined by: "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse
 * Transformers Run Like They Were Built for Hopper", section "TwELL: The
 * Packing Format That Fits the Machine" (fused MLP execution that packs the
 * up-projection's output without a separate pass over memory); "Nvidia and
 * Sakana make LLMs 30% faster by doing less math", section "Reshaping math
 * for the GPU" (sparse tokens on the fast path, rare dense tokens through a
 * dense matrix); "The Relentless Search for Efficiency in Large-Scale
 * Language Models", section "Mechanism of Action: Kernel-Level Optimization"
 * (the down-projection reads only the rows of active units).
 *   1. up-projection GEMM (MFMA for bf16) + bias + ReLU + rounding, whose
 *      epilogue packs each (row, tile) of h into TwELL and flags overflow
 *      (at most 64 rows: K is split over workgroups whose fp32 partial sums
 *      are added in a fixed order before the same epilogue; likewise for
 *      the fallback of step 4);
 *   2. row routing: a row with an overflowing tile is dense; dense rows are
 *      numbered in ascending order and copied to dense_values, their TwELL
 *      slots cleared;
 *   3. sparse down-projection of the TwELL rows: y[n] = sum over stored slots
 *      of value * w_down[t*tile + index];
 *   4. dense fallback GEMM for the dense rows: y[dense_rows[m]] =
 *      dense_values[m] W_down.
 * Steps 3 and 4 write disjoint rows of y and run one after the other on
 * `stream`.  For at most 64 rows step 3 may share a launch with step 4 (bf16)
 * or with step 2's dense-row build (float32, rows of at most 64 KB, when the
 * shape allows), computing the same bits as when it runs alone.
 * Arguments: shape (host pointer); x, w_up_t, b_up, w_down inputs; y output;
 * h_out (host pointer to a struct of device pointers) receives h in hybrid
 * TwELL form; h_dense_debug, if non-NULL, receives h [n_rows][d_ff] exactly
 * as packed (for bit-exact checks; costs one extra write of h); workspace /
 * workspace_bytes: scratch of at least ffn_sparse_workspace_size(shape)
 * bytes, never NULL (the routing writes it even for 0 rows), contents
 * undefined on entry and exit; d_status, if non-NULL, is set
 * on the device to TWELL_OK or TWELL_ERR_DENSE_CAPACITY.  On
 * TWELL_ERR_DENSE_CAPACITY the rows past dense_capacity are neither stored
 * nor computed, so y is undefined for them; *n_dense holds the true count so
 * the caller can retry with a larger dense buffer.  n_rows == 0 only sets
 * *n_dense = 0 and *d_status = TWELL_OK. */
int ffn_sparse_forward(const twell_shape* shape, const void* x, const void* w_up_t,
                       const float* b_up, const void* w_down, void* y,
                       const twell_hybrid* h_out, void* h_dense_debug, void* workspace,
                       size_t workspace_bytes, int32_t* d_status, void* stream);

/* The ReLU-gated layer, y = (ReLU(x W_gate + b_gate) * (x W_up + b_up)) W_down,
 * with its hidden activations h in hybrid TwELL form.  The pages describe
 * only the non-gated layer ("The Relentless Search for Efficiency in
 * Large-Scale Language Models", section "The Challenge of Sparsity Ignored by
 * GPUs": the sparsity comes from the ReLU); this is the same method applied to
 * the gated form of the sparse LLaMA models of "SakanaAI/sparser-faster-llms:
 * How TwELL Makes Sparse Transformers Run Like They Were Built for Hopper",
 * section "The Repo's Two Jobs".
 *   1-2. steps 1-2 of ffn_sparse_forward on the gate (w_gate_t, b_gate): the
 *        gate's activations ReLU(x W_gate + b_gate), rounded to the storage
 *        type, are packed and routed; their non-zeros fix h's stored places;
 *   2b.  at each stored place (row n, neuron j), the up branch
 *        u = x[n] . w_up_t[j] + b_up[j] (float32) is taken and h = g * u,
 *        rounded to the storage type, replaces the gate value g (u is computed
 *        only where the gate is non-zero);
 *   3-4. the hybrid down-projection of ffn_sparse_forward.
 * A place whose u is 0 keeps a stored 0.  w_up_t [d_ff][d_model] dtype and
 * b_up [d_ff] float32 as for the gate; the other arguments, the workspace
 * (ffn_sparse_workspace_size), the status word and the errors are those of
 * ffn_sparse_forward.  d_model up to 8192 (bf16) / 4096 (float32), else
 * TWELL_ERR_UNSUPPORTED. */
int ffn_sparse_gated_forward(const twell_shape* shape, const void* x, const void* w_gate_t,
                             const float* b_gate, const void* w_up_t, const float* b_up,
                             const void* w_down, void* y, const twell_hybrid* h_out,
                             void* workspace, size_t workspace_bytes, int32_t* d_status,
                             void* stream);

/* ffn_sparse_forward that also records five caller-created HIP events
 * (stage_events[0..4], hipEvent_t passed as void*) on `stream`: before step
 * 1 and after each of steps 1-4.  Every stage here runs in its own launches
 * (no step shares a launch with another), so a caller can time each stage
 * alone with hipEventElapsedTime.  Same arguments, results and errors as
 * ffn_sparse_forward; a NULL array or event is TWELL_ERR_INVALID_ARG.
 * Defined by the same passages as ffn_sparse_forward; the events are this
 * interface's own, for measurement. */
int ffn_sparse_forward_events(const twell_shape* shape, const void* x, const void* w_up_t,
                              const float* b_up, const void* w_down, void* y,
                              const twell_hybrid* h_out, void* h_dense_debug, void* workspace,
                              size_t workspace_bytes, int32_t* d_status, void* stream,
                              void* const* stage_events);

/* Bytes of device workspace twell_pack needs (0 for an invalid shape):
 * per-(row, tile) overflow flags and the row routing lists.  The scratch
 * behind dense_to_twell of "SakanaAI/sparser-faster-llms: How TwELL Makes
 * Sparse Transformers Run Like They Were Built for Hopper", section "TwELL:
 * The Packing Format That Fits the Machine". */
size_t twell_pack_workspace_size(const twell_shape* shape);

/* dense_to_twell: pack h [n_rows][d_ff] into the hybrid `out` under the
 * format rules above (same rules and same result as step 1-2 of
 * ffn_sparse_forward applied to h).
 * Defined by: "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse
 * Transformers Run Like They Were Built for Hopper", section "TwELL: The
 * Packing Format That Fits the Machine" (the dense-to-TwELL path); format and
 * row split per "Sparser, Faster, Lighter Transformer Language Models (Sakana
 * AI + NVIDIA)", Figure 1 description and packing-format flowchart.  Dense rows are copied bit for bit; in
 * sparse rows a -0.0 is dropped like +0.0.  workspace / d_status as for
 * ffn_sparse_forward. */
int twell_pack(const twell_shape* shape, const void* h, const twell_hybrid* out,
               void* workspace, size_t workspace_bytes, int32_t* d_status, void* stream);

/* Bytes of the fixed per-device scratch array behind twell_pack_noalloc. */
#define TWELL_NOALLOC_SCRATCH_BYTES (16u << 20)

/* twell_pack without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments
 * (minus the workspace), results and errors as twell_pack; the workspace is
 * a fixed array of TWELL_NOALLOC_SCRATCH_BYTES in the library's device code,
 * one per GPU, held until the process ends (its address is looked up once
 * per device, on the first call with that device current).  A shape whose
 * twell_pack_workspace_size exceeds TWELL_NOALLOC_SCRATCH_BYTES returns
 * TWELL_ERR_SCRATCH_LIMIT before anything is enqueued; so does a failure to
 * look the array up (TWELL_ERR_HIP).  Every call on one GPU shares its
 * array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Nothing in the array
 * needs to start at any value: each call writes every part it reads. */
int twell_pack_noalloc(const twell_shape* shape, const void* h, const twell_hybrid* out,
                       int32_t* d_status, void* stream);

/* twell_to_dense: h [n_rows][d_ff] = +0.0 everywhere, then every stored slot
 * (k < counts) is written to its column and every stored dense row
 * (the first min(*n_dense, dense_capacity) entries) is copied to its row.
 * dense_rows must be strictly ascending.
 * Defined by: "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse
 * Transformers Run Like They Were Built for Hopper", section "TwELL: The
 * Packing Format That Fits the Machine" (the TwELL-to-dense path); format per
 * "Sparser, Faster, Lighter Transformer Language Models (Sakana AI +
 * NVIDIA)", Figure 1 description. */
int twell_unpack(const twell_shape* shape, const twell_hybrid* in, void* h, void* stream);

/* The hybrid down-projection y [n_rows][d_model] = unpack(in) W_down:
 * TwELL rows by the sparse gather kernel, stored dense rows by the dense
 * fallback GEMM (float32 accumulation, one rounding at the end).  Every row
 * of y is written once: a row listed among the stored dense rows
 * (dense_rows[0 .. min(*n_dense, dense_capacity)), strictly ascending) by the
 * fallback only, every other row by the sparse kernel from its slots (a row
 * with no stored slot gets +0.0).  workspace / workspace_bytes: NULL / 0, or
 * a buffer of at least twell_spmm_workspace_size(shape) bytes for the dense
 * rows' split-K partial sums (smaller: TWELL_ERR_WORKSPACE; not 16-byte
 * aligned: TWELL_ERR_INVALID_ARG).  y is the same either way to within the
 * order of the fp32 additions of the dense rows.
 * Defined by: "The Relentless Search for Efficiency in Large-Scale Language
 * Models", section "Mechanism of Action: Kernel-Level Optimization" (only the
 * weight rows of non-zero activations are read); "Nvidia and Sakana make
 * LLMs 30% faster by doing less math", section "Reshaping math for the GPU"
 * (the dense matrix as a safety valve for overflowing tokens). */
int twell_spmm(const twell_shape* shape, const twell_hybrid* in, const void* w_down, void* y,
               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the optional twell_spmm workspace for this shape (0 when none
 * would be used; the call accepts NULL in any case).  Given, it holds the
 * fp32 partial sums of a split of the dense rows' K (d_ff) over many
 * workgroups, as the forward's own fallback does: at most 64 rows, the
 * split-K kernels; bf16 past that, up to 32 K slices of the live rows, at
 * most 32 MiB.  Without it the fallback runs one workgroup per output tile
 * over the whole of K, which leaves most of the GPU idle when there are few
 * dense rows.  Any 16-byte-aligned device buffer of at least this size;
 * its contents are scratch, and calls that share one on one GPU race. */
size_t twell_spmm_workspace_size(const twell_shape* shape);

/* ---- ELL rows: Figure 1(a) beside TwELL (Figure 1(b)) and the hybrid
 * (Figure 1(c)) of "Sparser, Faster, Lighter Transformer Language Models
 * (Sakana AI + NVIDIA)", Figure 1 description.  Each token row keeps its
 * non-zeros in ascending column order in the first `counts` of `width`
 * slots, with their 16-bit column numbers; padding slots hold +0.0 and
 * column 0.  It is TwELL with one tile spanning the whole row, so a twell_shape
 * describes it with tile == d_ff and capacity == width (1 <= width <=
 * min(d_ff, 65535)); d_ff must be a multiple of 8 and at most 65536.  A row
 * with more than `width` non-zeros goes to the dense matrix exactly as a row
 * with an overflowing tile does in the hybrid TwELL ("Nvidia and Sakana make
 * LLMs 30% faster by doing less math", section "Reshaping math for the GPU").
 * Slot positions depend on the whole row, so ELL is packed from a
 * materialised h, not from the tiled up-projection's epilogue. */
typedef struct twell_ell {
  void* values;          /* [n_rows][width] dtype */
  uint16_t* columns;     /* [n_rows][width] uint16 column in [0, d_ff) */
  uint16_t* counts;      /* [n_rows] uint16 non-zeros stored (0 for dense rows) */
  int32_t* dense_rows;   /* [dense_capacity] int32, ascending token rows */
  void* dense_values;    /* [dense_capacity][d_ff] dtype, the dense rows bit for bit */
  int32_t* n_dense;      /* device int32: number of dense rows (as in twell_hybrid) */
  int64_t dense_capacity;
} twell_ell;

/* Bytes of device workspace ell_pack needs (0 for an invalid shape): one
 * overflow flag per row and the row routing lists. */
size_t ell_pack_workspace_size(const twell_shape* shape);

/* dense_to_ell: pack h [n_rows][d_ff] into `out` (shape: tile == d_ff,
 * capacity == width).  Same routing, dense-row copy, status word and
 * capacity behaviour as twell_pack; -0.0 is dropped like +0.0 in sparse
 * rows.  Defined by the Figure 1 description (panel a) cited above. */
int ell_pack(const twell_shape* shape, const void* h, const twell_ell* out, void* workspace,
             size_t workspace_bytes, int32_t* d_status, void* stream);

/* ell_to_dense: h [n_rows][d_ff] = +0.0 everywhere, then the first counts[n]
 * slots of each row at their columns, and each stored dense row copied
 * (dense_rows strictly ascending).  Rows of more than 64 KB are
 * TWELL_ERR_UNSUPPORTED.  Defined by the Figure 1 description (panel a). */
int ell_unpack(const twell_shape* shape, const twell_ell* in, void* h, void* stream);

/* The ELL down-projection y [n_rows][d_model] = ell_to_dense(in) W_down, every
 * row written once: rows listed among the stored dense rows by the dense
 * fallback GEMM, the others from their slots (float32 accumulation, one
 * rounding).  Defined by the Figure 1 description (panel a) and "The
 * Relentless Search for Efficiency in Large-Scale Language Models", section
 * "Mechanism of Action: Kernel-Level Optimization" (only the weight rows of
 * non-zero activations are read). */
int ell_spmm(const twell_shape* shape, const twell_ell* in, const void* w_down, void* y,
             void* stream);

/* ---- The layer's backward pass.  "Sparser, Faster, Lighter Transformer
 * Language Models (Sakana AI + NVIDIA)" (TL;DR and Figure 1 description)
 * carries the sparse format into training as well as inference; "Nvidia and
 * Sakana make LLMs 30% faster by doing less math", section "More speed, less
 * power, zero quality loss", reports the training-side speed and peak-memory
 * gains.  The pages do not write the gradients out; they follow from the
 * forward y = ReLU(x W_up + b_up) W_down by the chain rule, with the ReLU's
 * derivative read from the stored h (1 where h != 0, 0 elsewhere; at a
 * pre-activation of exactly 0 the derivative is taken as 0, the usual
 * convention). */

/* Bytes of device workspace ffn_sparse_backward needs for this shape and a
 * hybrid h with `dense_capacity` dense-row slots (0 for an invalid shape or
 * when the per-neuron lists would hold more than 2^31 - 1 entries or d_model
 * is past the backward's limit): dz in
 * h's slots and in its dense rows, a (neuron, row) bitmap of h's non-zeros
 * with its word prefixes, one flag per row, and one 16-byte entry per TwELL
 * slot and per stored dense element. */
size_t ffn_sparse_backward_workspace_size(const twell_shape* shape, int64_t dense_capacity);

/* Gradients of L = sum(y * dy) for y = ReLU(x W_up + b_up) W_down, from the
 * stored hidden activations h (the hybrid that ffn_sparse_forward or
 * twell_pack wrote for the same x, weights and shape):
 *   dz      = dy W_down^T at the non-zeros of h (0 elsewhere), rounded to
 *             the storage type;
 *   dw_down = h^T dy                  [d_ff][d_model] float32
 *   dw_up_t = dz^T x (W_up transposed) [d_ff][d_model] float32
 *   db_up   = column sums of dz        [d_ff] float32
 *   dx      = dz W_up (= dz w_up_t)    [n_rows][d_model] dtype
 * Each weight and bias gradient element is one float32 sum over the rows
 * where h is non-zero, in ascending row order; the results do not depend on
 * scheduling and are written, not added to (the caller accumulates over
 * micro-batches).  dx is the hybrid product of twell_spmm with dz's values
 * in h's slots and rows.  A row listed among the stored dense rows is read
 * from dense_values only; after a TWELL_ERR_DENSE_CAPACITY forward the rows
 * past dense_capacity hold no non-zero, so they contribute nothing and get
 * dx = 0.
 * d_model is at most 16384 (bf16) or 8192 (float32), else
 * TWELL_ERR_UNSUPPORTED.
 * Arguments: shape (host pointer; the forward's shape); x, w_up_t, w_down,
 * dy [n_rows][d_model] inputs in dtype; h (host pointer to device pointers)
 * the stored activations; dx, dw_up_t, db_up, dw_down outputs; workspace of
 * at least ffn_sparse_backward_workspace_size(shape, h->dense_capacity)
 * bytes, never NULL, contents undefined on entry and exit.  n_rows == 0
 * writes zero weight and bias gradients. */
int ffn_sparse_backward(const twell_shape* shape, const void* x, const void* w_up_t,
                        const void* w_down, const twell_hybrid* h, const void* dy, void* dx,
                        float* dw_up_t, float* db_up, float* dw_down, void* workspace,
                        size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
