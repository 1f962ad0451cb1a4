"""CPU oracle for the hybrid-TwELL ReLU FFN forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
module imports nothing from the product path.

Everything here is plain and slow on purpose: NumPy in float64 for the
arithmetic, pure-Python loops for the reference packer, and library primitives
(dense matmul, a sparse-times-dense product) only as whole steps.

Sources (the web pages on "Sparser, Faster, Lighter Transformer Language
Models", Sakana AI + NVIDIA):

* [blog] "The Relentless Search for Efficiency in Large-Scale Language Models",
  section "The Challenge of Sparsity Ignored by GPUs": a hidden unit of the FFN
  is active when it is non-zero after the activation function (ReLU).
* [wiki] "Sparser, Faster, Lighter Transformer Language Models (Sakana AI +
  NVIDIA)", Figure 1 description and the packing-format flowchart: a values
  array holding the non-zeros only, an indices array of tile-local positions,
  per-tile non-zero counts, tile size T and tile index t; the hybrid variant
  splits rows between formats according to how their non-zeros distribute.
* [news] "Nvidia and Sakana make LLMs 30% faster by doing less math", section
  "Reshaping math for the GPU": the rare dense tokens that cannot be skipped go
  to a dense matrix that acts as a safety valve.
* [repo] "SakanaAI/sparser-faster-llms: How TwELL Makes Sparse Transformers Run
  Like They Were Built for Hopper", section "TwELL: The Packing Format That
  Fits the Machine": the kernel layer converts dense-to-TwELL and
  TwELL-to-dense and runs the fused MLP.

Readings taken where the pages are silent (each is also listed in the design
notes):

* FFN form: y = ReLU(x W_up + b) W_down, non-gated, no down-projection bias.
* Tile t of a token row is columns [t*T, (t+1)*T); d_ff must be a multiple of T.
* Inside a tile the non-zeros are kept in ascending column order; slot k holds
  the k-th non-zero.
* A tile fits when its count is <= C; it overflows when count > C.
* Routing is per row: one overflowing tile sends the whole token row to the
  dense matrix.  Dense rows keep count 0 and all-padding slots in the TwELL
  arrays, and are listed in ascending token order.
* Padding slots hold value +0.0 (all-zero bits) and index 0.
* "Non-zero" is tested by value on the stored (already rounded) number: -0.0
  is zero, NaN is non-zero.
* Indices and counts are uint8 (T <= 256, C <= 255).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import scipy.sparse


# --------------------------------------------------------------------------
# Storage-dtype decoding
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float32.

    A bfloat16 number is the upper half of the float32 with the same sign,
    exponent and leading 7 mantissa bits, so decoding is a 16-bit left shift.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# --------------------------------------------------------------------------
# Dense FFN (the plain definition) [blog], [wiki "What it claims"]
# --------------------------------------------------------------------------
def ffn_hidden(x: np.ndarray, w_up_t: np.ndarray, b_up: np.ndarray) -> np.ndarray:
    """h = ReLU(x @ W_up + b) in float64, unrounded.

    ``w_up_t`` is W_up stored transposed, [d_ff, d_model], so z[n, j] =
    sum_i x[n, i] * w_up_t[j, i] + b[j].  ReLU keeps z where z > 0, else 0.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_up_t, dtype=np.float64)
    b = np.asarray(b_up, dtype=np.float64)
    z = x @ w.T + b[None, :]
    return np.where(z > 0.0, z, 0.0)


def ffn_forward(x, w_up_t, b_up, w_down):
    """Return (h, y) of the dense FFN in float64: y = h @ W_down, W_down [d_ff, d_model]."""
    h = ffn_hidden(x, w_up_t, b_up)
    y = h @ np.asarray(w_down, dtype=np.float64)
    return h, y


def ffn_forward_rows(x, w_up_t, b_up, w_down, rows):
    """The dense FFN on a subset of token rows (rows are independent)."""
    rows = np.asarray(rows, dtype=np.int64)
    return ffn_forward(np.asarray(x)[rows], w_up_t, b_up, w_down)


# --------------------------------------------------------------------------
# Hybrid TwELL [wiki Figure 1], [news "Reshaping math for the GPU"]
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Hybrid:
    """A token-row matrix h [N, d_ff] in hybrid TwELL form.

    values  [N, nt, C]  storage-dtype numbers (a float NumPy dtype here)
    indices [N, nt, C]  uint8 tile-local column of each slot
    counts  [N, nt]     uint8 non-zeros stored in each tile
    dense_rows   [n_dense]        int32 token rows kept dense, ascending
    dense_values [n_dense, d_ff]  those rows, copied bit for bit
    """

    tile: int
    capacity: int
    d_ff: int
    values: np.ndarray
    indices: np.ndarray
    counts: np.ndarray
    dense_rows: np.ndarray
    dense_values: np.ndarray

    @property
    def n_rows(self) -> int:
        return self.counts.shape[0]

    @property
    def n_tiles(self) -> int:
        return self.d_ff // self.tile

    @property
    def n_dense(self) -> int:
        return int(self.dense_rows.shape[0])


def _check_geometry(d_ff: int, tile: int, capacity: int) -> None:
    if tile < 1 or tile > 256 or d_ff % tile != 0:
        raise ValueError(f"tile {tile} must be in [1, 256] and divide d_ff {d_ff}")
    if capacity < 1 or capacity > min(tile, 255):
        raise ValueError(f"capacity {capacity} must be in [1, min(T, 255)]")


def pack_reference(h: np.ndarray, tile: int, capacity: int) -> Hybrid:
    """dense_to_twell by its definition, one row, tile and column at a time.

    For small inputs only (pure-Python loops).
    """
    h = np.asarray(h)
    n, d_ff = h.shape
    _check_geometry(d_ff, tile, capacity)
    nt = d_ff // tile
    values = np.zeros((n, nt, capacity), dtype=h.dtype)
    indices = np.zeros((n, nt, capacity), dtype=np.uint8)
    counts = np.zeros((n, nt), dtype=np.uint8)
    dense_rows = []
    for r in range(n):
        tiles = []
        for t in range(nt):
            entries = []
            for c in range(t * tile, (t + 1) * tile):
                v = h[r, c]
                if v != 0:  # -0.0 == 0 is zero; NaN != 0 is non-zero
                    entries.append((c - t * tile, v))
            tiles.append(entries)
        if any(len(e) > capacity for e in tiles):
            dense_rows.append(r)  # whole row to the dense matrix
            continue
        for t, entries in enumerate(tiles):
            counts[r, t] = len(entries)
            for k, (local, v) in enumerate(entries):
                indices[r, t, k] = local
                values[r, t, k] = v
    dense_rows = np.array(dense_rows, dtype=np.int32)
    dense_values = h[dense_rows].copy() if len(dense_rows) else np.zeros((0, d_ff), h.dtype)
    return Hybrid(tile, capacity, d_ff, values, indices, counts, dense_rows, dense_values)


def tile_counts(h: np.ndarray, tile: int) -> np.ndarray:
    """Non-zeros per (row, tile): [N, nt] int64."""
    n, d_ff = h.shape
    return (np.asarray(h).reshape(n, d_ff // tile, tile) != 0).sum(axis=-1)


def pack(h: np.ndarray, tile: int, capacity: int, chunk_rows: int = 1024) -> Hybrid:
    """dense_to_twell, vectorized over rows in chunks (same result as pack_reference)."""
    h = np.asarray(h)
    n, d_ff = h.shape
    _check_geometry(d_ff, tile, capacity)
    nt = d_ff // tile
    values = np.zeros((n, nt, capacity), dtype=h.dtype)
    indices = np.zeros((n, nt, capacity), dtype=np.uint8)
    counts = np.zeros((n, nt), dtype=np.uint8)
    dense_mask = np.zeros(n, dtype=bool)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        hv = h[r0:r1].reshape(r1 - r0, nt, tile)
        nz = hv != 0
        cnt = nz.sum(axis=-1)
        dense = (cnt > capacity).any(axis=-1)
        dense_mask[r0:r1] = dense
        slot = np.cumsum(nz, axis=-1) - 1  # rank of each non-zero inside its tile
        keep = nz & ~dense[:, None, None]
        rr, tt, cc = np.nonzero(keep)
        kk = slot[rr, tt, cc]
        values[r0 + rr, tt, kk] = hv[rr, tt, cc]
        indices[r0 + rr, tt, kk] = cc.astype(np.uint8)
        counts[r0:r1] = np.where(dense[:, None], 0, cnt).astype(np.uint8)
    dense_rows = np.nonzero(dense_mask)[0].astype(np.int32)
    dense_values = h[dense_rows].copy()
    return Hybrid(tile, capacity, d_ff, values, indices, counts, dense_rows, dense_values)


def unpack(hyb: Hybrid) -> np.ndarray:
    """twell_to_dense: +0 everywhere, then scatter the slots and copy the dense rows."""
    n, nt, cap = hyb.values.shape
    h = np.zeros((n, hyb.d_ff), dtype=hyb.values.dtype)
    for t in range(nt):
        for k in range(cap):
            live = np.nonzero(hyb.counts[:, t] > k)[0]
            h[live, t * hyb.tile + hyb.indices[live, t, k].astype(np.int64)] = hyb.values[live, t, k]
    if hyb.n_dense:
        h[hyb.dense_rows] = hyb.dense_values
    return h


def to_csr(hyb: Hybrid) -> scipy.sparse.csr_matrix:
    """The TwELL part (sparse rows only) as a float64 CSR matrix [N, d_ff]."""
    n, nt, cap = hyb.values.shape
    k = np.arange(cap)[None, None, :]
    live = k < hyb.counts[:, :, None].astype(np.int64)
    rr, tt, kk = np.nonzero(live)
    cols = tt * hyb.tile + hyb.indices[rr, tt, kk].astype(np.int64)
    vals = hyb.values[rr, tt, kk].astype(np.float64)
    return scipy.sparse.csr_matrix((vals, (rr, cols)), shape=(n, hyb.d_ff))


def spmm(hyb: Hybrid, w_down: np.ndarray) -> np.ndarray:
    """Hybrid down-projection y = h @ W_down in float64, read from the hybrid arrays.

    Sparse rows: y[n] = sum_t sum_{k < counts[n,t]} values[n,t,k] * W_down[t*T + indices[n,t,k]].
    Dense rows:  y[dense_rows[m]] = dense_values[m] @ W_down.
    """
    w = np.asarray(w_down, dtype=np.float64)
    y = np.asarray(to_csr(hyb) @ w, dtype=np.float64)
    if hyb.n_dense:
        y[hyb.dense_rows] = hyb.dense_values.astype(np.float64) @ w
    return y


# --------------------------------------------------------------------------
# Textbook ELLPACK (Figure 1(a)), used as an independent pin for T = d_ff
# --------------------------------------------------------------------------
def ell_pack_textbook(h: np.ndarray, width: int):
    """Classic ELLPACK of a dense matrix: per row, the non-zeros in column
    order padded to ``width`` slots, with their column numbers.

    Returns (values [N, width], columns [N, width] int64, row_nnz [N]).
    Raises ValueError when a row holds more than ``width`` non-zeros.
    """
    h = np.asarray(h)
    n, m = h.shape
    vals = np.zeros((n, width), dtype=h.dtype)
    cols = np.zeros((n, width), dtype=np.int64)
    nnz = np.zeros(n, dtype=np.int64)
    for r in range(n):
        nzc = [c for c in range(m) if h[r, c] != 0]
        if len(nzc) > width:
            raise ValueError(f"row {r} has {len(nzc)} non-zeros > width {width}")
        nnz[r] = len(nzc)
        for k, c in enumerate(nzc):
            vals[r, k] = h[r, c]
            cols[r, k] = c
    return vals, cols, nnz


# --------------------------------------------------------------------------
# ELL rows with the hybrid split: Figure 1(a) beside TwELL [wiki Figure 1]
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Ell:
    """A token-row matrix h [N, d_ff] as ELL rows plus dense rows.

    values  [N, width]  the row's non-zeros in ascending column order, then +0
    columns [N, width]  int64 column of each slot (0 in padding)
    counts  [N]         int64 non-zeros stored (0 for a dense row)
    dense_rows   [n_dense]        int32 rows with more than `width` non-zeros
    dense_values [n_dense, d_ff]  those rows, copied bit for bit
    """

    width: int
    d_ff: int
    values: np.ndarray
    columns: np.ndarray
    counts: np.ndarray
    dense_rows: np.ndarray
    dense_values: np.ndarray

    @property
    def n_dense(self) -> int:
        return int(self.dense_rows.shape[0])


def ell_pack(h: np.ndarray, width: int) -> Ell:
    """dense_to_ell by its definition, one row and column at a time.

    A row keeps its non-zeros (tested by value, so -0.0 is zero and NaN is
    not) in ascending column order in its first slots, padding after them;
    a row with more than ``width`` non-zeros goes to the dense matrix whole,
    the hybrid rule with one tile spanning the row.  Pure-Python loops: for
    small inputs.
    """
    h = np.asarray(h)
    n, d_ff = h.shape
    if width < 1 or width > d_ff:
        raise ValueError(f"width {width} must be in [1, d_ff]")
    values = np.zeros((n, width), dtype=h.dtype)
    columns = np.zeros((n, width), dtype=np.int64)
    counts = np.zeros(n, dtype=np.int64)
    dense_rows = []
    for r in range(n):
        nz = [c for c in range(d_ff) if h[r, c] != 0]
        if len(nz) > width:
            dense_rows.append(r)
            continue
        counts[r] = len(nz)
        for k, c in enumerate(nz):
            values[r, k] = h[r, c]
            columns[r, k] = c
    dense_rows = np.array(dense_rows, dtype=np.int32)
    dense_values = h[dense_rows].copy() if len(dense_rows) else np.zeros((0, d_ff), h.dtype)
    return Ell(width, d_ff, values, columns, counts, dense_rows, dense_values)


def ell_unpack(e: Ell) -> np.ndarray:
    """ell_to_dense: +0 everywhere, the first counts[n] slots of each row at their
    columns, then the dense rows copied."""
    n = e.counts.shape[0]
    h = np.zeros((n, e.d_ff), dtype=e.values.dtype)
    for r in range(n):
        for k in range(int(e.counts[r])):
            h[r, int(e.columns[r, k])] = e.values[r, k]
    if e.n_dense:
        h[e.dense_rows] = e.dense_values
    return h


# --------------------------------------------------------------------------
# ReLU-gated FFN (GLU form).  The pages describe only the non-gated layer; the
# gated form is this oracle's extension, for LLaMA-style FFNs [repo "The
# Repo's Two Jobs": a sparse LLaMA model], with its sparsity taken from the
# ReLU of the gate exactly as the plain layer takes it from its ReLU [blog
# "The Challenge of Sparsity Ignored by GPUs"].
# --------------------------------------------------------------------------
def gated_ffn_hidden(x, w_gate_t, b_gate, w_up_t, b_up) -> np.ndarray:
    """h = ReLU(x W_gate + b_gate) * (x W_up + b_up), elementwise, in float64.

    Both weights are stored transposed, [d_ff, d_model].  h is zero wherever
    the gate's pre-activation is <= 0, whatever the up branch holds.
    """
    x = np.asarray(x, dtype=np.float64)
    zg = x @ np.asarray(w_gate_t, dtype=np.float64).T + np.asarray(b_gate, dtype=np.float64)[None, :]
    zu = x @ np.asarray(w_up_t, dtype=np.float64).T + np.asarray(b_up, dtype=np.float64)[None, :]
    return np.where(zg > 0.0, zg, 0.0) * zu


def gated_ffn_forward(x, w_gate_t, b_gate, w_up_t, b_up, w_down):
    """Return (h, y) of the gated FFN in float64: y = h @ W_down."""
    h = gated_ffn_hidden(x, w_gate_t, b_gate, w_up_t, b_up)
    return h, h @ np.asarray(w_down, dtype=np.float64)


# --------------------------------------------------------------------------
# Training step: the gradients of the layer [wiki TL;DR: inference and
# training], [news "More speed, less power, zero quality loss"]
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Grads:
    """Gradients of the scalar L = sum(y * dy) for y = ReLU(x W_up + b) W_down."""

    dx: np.ndarray       # [N, d_model]
    dw_up_t: np.ndarray  # [d_ff, d_model]
    db: np.ndarray       # [d_ff]
    dw_down: np.ndarray  # [d_ff, d_model]


def ffn_backward_from_h(x, h, w_up_t, w_down, dy) -> Grads:
    """Backward pass from the stored activations h, in float64.

    The ReLU passes gradient exactly where the stored activation is non-zero,
    so every gradient is read from the non-zeros of h:
      dW_down = h^T dy
      dz      = (dy W_down^T) masked to h != 0
      db      = column sums of dz
      dW_up^T = dz^T x
      dx      = dz W_up^T (W_up stored transposed: dz @ w_up_t)
    """
    x = np.asarray(x, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    w_up_t = np.asarray(w_up_t, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    dw_down = h.T @ dy
    dz = np.where(h != 0, dy @ w_down.T, 0.0)
    return Grads(dx=dz @ w_up_t, dw_up_t=dz.T @ x, db=dz.sum(axis=0), dw_down=dw_down)


def ffn_backward(x, w_up_t, b_up, w_down, dy) -> Grads:
    """Backward pass of the dense FFN: h from the forward definition, then
    ffn_backward_from_h."""
    return ffn_backward_from_h(x, ffn_hidden(x, w_up_t, b_up), w_up_t, w_down, dy)


def sampled_dots(hyb: Hybrid, a: np.ndarray, b: np.ndarray):
    """The product a b^T sampled where the hybrid stores a non-zero, in float64.

    For every live slot (n, t, k): sum_c a[n, c] * b[t*T + indices[n,t,k], c],
    in the slot's place of a [N, nt, C] array (0 elsewhere); for every stored
    dense row m: the same dot at each column j where dense_values[m, j] != 0
    (0 elsewhere), in a [n_dense, d_ff] array.  For the backward this is dz
    (a = dy, b = W_down) at the positions the ReLU lets through.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n, nt, cap = hyb.values.shape
    vals = np.zeros((n, nt, cap))
    for t in range(nt):
        for k in range(cap):
            live = np.nonzero(hyb.counts[:, t] > k)[0]
            if len(live):
                cols = t * hyb.tile + hyb.indices[live, t, k].astype(np.int64)
                vals[live, t, k] = np.einsum("nc,nc->n", a[live], b[cols])
    dense = np.zeros((hyb.n_dense, hyb.d_ff))
    for m in range(hyb.n_dense):
        nzc = np.nonzero(hyb.dense_values[m] != 0)[0]
        dense[m, nzc] = b[nzc] @ a[hyb.dense_rows[m]]
    return vals, dense
