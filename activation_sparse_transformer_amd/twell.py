"""Python binding of libtwell.so (ctypes over the C ABI in include/twell.h).

This layer only marshals arguments: it checks tensor placement and types,
allocates output / workspace tensors through PyTorch when the caller does not
pass them, and hands raw device pointers plus the current HIP stream to the
library.  Every step of the forward pass runs in the library's HIP kernels;
there is no fallback of any kind, so a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtwell.so")

TWELL_OK = 0
TWELL_ERR_INVALID_ARG = -1
TWELL_ERR_UNSUPPORTED = -2
TWELL_ERR_WORKSPACE = -3
TWELL_ERR_HIP = -4
TWELL_ERR_DENSE_CAPACITY = -5
TWELL_ERR_SCRATCH_LIMIT = -6
NOALLOC_SCRATCH_BYTES = 16 << 20  # TWELL_NOALLOC_SCRATCH_BYTES

_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}

EXPORTS = (
    "twell_version", "twell_status_string", "ffn_sparse_workspace_size", "ffn_sparse_forward",
    "ffn_sparse_forward_events", "twell_pack_workspace_size", "twell_pack", "twell_pack_noalloc",
    "twell_unpack", "twell_spmm", "twell_spmm_workspace_size", "ell_pack_workspace_size",
    "ell_pack", "ell_unpack", "ell_spmm",
    "ffn_sparse_backward_workspace_size", "ffn_sparse_backward", "ffn_sparse_gated_forward",
)


class TwellError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


class Shape(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("tile", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class HybridStruct(ctypes.Structure):
    _fields_ = [
        ("values", ctypes.c_void_p), ("indices", ctypes.c_void_p), ("counts", ctypes.c_void_p),
        ("dense_rows", ctypes.c_void_p), ("dense_values", ctypes.c_void_p),
        ("n_dense", ctypes.c_void_p), ("dense_capacity", ctypes.c_int64),
    ]


class EllStruct(ctypes.Structure):
    _fields_ = [
        ("values", ctypes.c_void_p), ("columns", ctypes.c_void_p), ("counts", ctypes.c_void_p),
        ("dense_rows", ctypes.c_void_p), ("dense_values", ctypes.c_void_p),
        ("n_dense", ctypes.c_void_p), ("dense_capacity", ctypes.c_int64),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtwell.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m activation_sparse_transformer_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int
    H = ctypes.POINTER(HybridStruct)
    sz = ctypes.c_size_t
    lib.twell_version.argtypes, lib.twell_version.restype = [], I
    lib.twell_status_string.argtypes, lib.twell_status_string.restype = [I], ctypes.c_char_p
    lib.ffn_sparse_workspace_size.argtypes, lib.ffn_sparse_workspace_size.restype = [S], sz
    lib.twell_pack_workspace_size.argtypes, lib.twell_pack_workspace_size.restype = [S], sz
    lib.ffn_sparse_forward.argtypes = [S, P, P, P, P, P, H, P, P, sz, P, P]
    lib.ffn_sparse_forward.restype = I
    lib.ffn_sparse_forward_events.argtypes = [S, P, P, P, P, P, H, P, P, sz, P, P, P]
    lib.ffn_sparse_forward_events.restype = I
    lib.ffn_sparse_gated_forward.argtypes = [S, P, P, P, P, P, P, P, H, P, sz, P, P]
    lib.ffn_sparse_gated_forward.restype = I
    lib.twell_pack.argtypes, lib.twell_pack.restype = [S, P, H, P, sz, P, P], I
    lib.twell_pack_noalloc.argtypes, lib.twell_pack_noalloc.restype = [S, P, H, P, P], I
    lib.twell_unpack.argtypes, lib.twell_unpack.restype = [S, H, P, P], I
    lib.twell_spmm.argtypes, lib.twell_spmm.restype = [S, H, P, P, P, sz, P], I
    lib.twell_spmm_workspace_size.argtypes, lib.twell_spmm_workspace_size.restype = [S], sz
    E = ctypes.POINTER(EllStruct)
    lib.ell_pack_workspace_size.argtypes, lib.ell_pack_workspace_size.restype = [S], sz
    lib.ell_pack.argtypes, lib.ell_pack.restype = [S, P, E, P, sz, P, P], I
    lib.ell_unpack.argtypes, lib.ell_unpack.restype = [S, E, P, P], I
    lib.ell_spmm.argtypes, lib.ell_spmm.restype = [S, E, P, P, P], I
    i64 = ctypes.c_int64
    lib.ffn_sparse_backward_workspace_size.argtypes = [S, i64]
    lib.ffn_sparse_backward_workspace_size.restype = sz
    lib.ffn_sparse_backward.argtypes = [S, P, P, P, H, P, P, P, P, P, P, sz, P]
    lib.ffn_sparse_backward.restype = I
    _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return load().twell_status_string(int(code)).decode()
    except RuntimeError:
        return f"status {code}"


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(code: int, where: str) -> None:
    if code != TWELL_OK:
        raise TwellError(code, where)


def _need(t: torch.Tensor, name: str, device, dtype=None, shape=None) -> None:
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_shape(n_rows: int, d_model: int, d_ff: int, tile: int, capacity: int,
               dtype: torch.dtype) -> Shape:
    if dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype {dtype} is not supported (float32 or bfloat16)")
    return Shape(n_rows, d_model, d_ff, tile, capacity, _DTYPE_CODE[dtype], 0)


@dataclasses.dataclass
class Hybrid:
    """Device tensors of one hybrid TwELL matrix (see twell_hybrid in twell.h)."""

    tile: int
    capacity: int
    d_ff: int
    values: torch.Tensor        # [N, nt, C] dtype
    indices: torch.Tensor       # [N, nt, C] uint8
    counts: torch.Tensor        # [N, nt] uint8
    dense_rows: torch.Tensor    # [dense_capacity] int32
    dense_values: torch.Tensor  # [dense_capacity, d_ff] dtype
    n_dense: torch.Tensor       # [1] int32

    @property
    def n_rows(self) -> int:
        return self.counts.shape[0]

    @property
    def dense_capacity(self) -> int:
        return self.dense_rows.shape[0]

    @property
    def dtype(self) -> torch.dtype:
        return self.values.dtype

    @classmethod
    def empty(cls, n_rows: int, d_ff: int, tile: int, capacity: int, dtype: torch.dtype,
              device, dense_capacity: Optional[int] = None) -> "Hybrid":
        if d_ff % tile:
            raise ValueError(f"tile {tile} must divide d_ff {d_ff}")
        nt = d_ff // tile
        cap = n_rows if dense_capacity is None else dense_capacity
        return cls(
            tile, capacity, d_ff,
            torch.empty((n_rows, nt, capacity), dtype=dtype, device=device),
            torch.empty((n_rows, nt, capacity), dtype=torch.uint8, device=device),
            torch.empty((n_rows, nt), dtype=torch.uint8, device=device),
            torch.empty((cap,), dtype=torch.int32, device=device),
            torch.empty((cap, d_ff), dtype=dtype, device=device),
            torch.empty((1,), dtype=torch.int32, device=device),
        )

    def struct(self) -> HybridStruct:
        return HybridStruct(
            _ptr(self.values), _ptr(self.indices), _ptr(self.counts), _ptr(self.dense_rows),
            _ptr(self.dense_values), _ptr(self.n_dense), self.dense_capacity)

    def validate(self, device) -> None:
        n, nt, C = self.n_rows, self.d_ff // self.tile, self.capacity
        _need(self.values, "values", device, shape=(n, nt, C))
        _need(self.indices, "indices", device, torch.uint8, (n, nt, C))
        _need(self.counts, "counts", device, torch.uint8, (n, nt))
        _need(self.dense_rows, "dense_rows", device, torch.int32)
        _need(self.dense_values, "dense_values", device, self.values.dtype,
              (self.dense_capacity, self.d_ff))
        _need(self.n_dense, "n_dense", device, torch.int32, (1,))

    def n_dense_host(self) -> int:
        return int(self.n_dense.item())


def ffn_workspace_bytes(shape: Shape) -> int:
    return int(load().ffn_sparse_workspace_size(ctypes.byref(shape)))


def pack_workspace_bytes(shape: Shape) -> int:
    return int(load().twell_pack_workspace_size(ctypes.byref(shape)))


@dataclasses.dataclass
class ForwardBuffers:
    """Everything ffn_sparse_forward writes, allocated once for reuse."""

    y: torch.Tensor
    hybrid: Hybrid
    workspace: torch.Tensor
    status: torch.Tensor
    h_debug: Optional[torch.Tensor] = None


def forward_buffers(n_rows: int, d_model: int, d_ff: int, tile: int, capacity: int,
                    dtype: torch.dtype, device, dense_capacity: Optional[int] = None,
                    debug_h: bool = False) -> ForwardBuffers:
    shape = make_shape(n_rows, d_model, d_ff, tile, capacity, dtype)
    ws = ffn_workspace_bytes(shape)
    if ws == 0 and n_rows > 0:
        raise TwellError(TWELL_ERR_INVALID_ARG, "ffn_sparse_workspace_size")
    return ForwardBuffers(
        y=torch.empty((n_rows, d_model), dtype=dtype, device=device),
        hybrid=Hybrid.empty(n_rows, d_ff, tile, capacity, dtype, device, dense_capacity),
        workspace=torch.empty((max(ws, 1),), dtype=torch.uint8, device=device),
        status=torch.empty((1,), dtype=torch.int32, device=device),
        h_debug=torch.empty((n_rows, d_ff), dtype=dtype, device=device) if debug_h else None,
    )


def ffn_sparse_forward(x: torch.Tensor, w_up_t: torch.Tensor, b_up: torch.Tensor,
                       w_down: torch.Tensor, tile: int, capacity: int, *,
                       dense_capacity: Optional[int] = None, debug_h: bool = False,
                       out: Optional[ForwardBuffers] = None,
                       stage_events: Optional[list] = None) -> ForwardBuffers:
    """y = ReLU(x @ w_up_t.T + b_up) @ w_down with h produced in hybrid TwELL form.

    x [N, d_model]; w_up_t, w_down [d_ff, d_model]; b_up [d_ff] float32.
    Returns the ForwardBuffers holding y, the hybrid h, the device status word
    and (with debug_h) the dense h exactly as packed.  Asynchronous: read
    results after the current stream reaches them.  ``stage_events``: five
    torch.cuda.Event(enable_timing=True) recorded before the up-projection and
    after each of the four stages (up+pack, routing, sparse product, dense
    fallback) on the current stream.
    """
    dev = x.device
    n, dm = x.shape
    dff = w_up_t.shape[0]
    dt = x.dtype
    _need(x, "x", dev, dt)
    _need(w_up_t, "w_up_t", dev, dt, (dff, dm))
    _need(b_up, "b_up", dev, torch.float32, (dff,))
    _need(w_down, "w_down", dev, dt, (dff, dm))
    if out is None:
        out = forward_buffers(n, dm, dff, tile, capacity, dt, dev, dense_capacity, debug_h)
    shape = make_shape(n, dm, dff, tile, capacity, dt)
    _need(out.y, "y", dev, dt, (n, dm))
    out.hybrid.validate(dev)
    if out.h_debug is not None:
        _need(out.h_debug, "h_debug", dev, dt, (n, dff))
    hs = out.hybrid.struct()
    args = (ctypes.byref(shape), _ptr(x), _ptr(w_up_t), _ptr(b_up), _ptr(w_down), _ptr(out.y),
            ctypes.byref(hs), _ptr(out.h_debug), _ptr(out.workspace), out.workspace.numel(),
            _ptr(out.status), _stream(dev))
    if stage_events is None:
        code = load().ffn_sparse_forward(*args)
    else:
        if len(stage_events) != 5:
            raise ValueError("stage_events needs five events")
        for e in stage_events:
            if not e.cuda_event:
                e.record()  # creates the underlying event; re-recorded inside the call
        arr = (ctypes.c_void_p * 5)(*[e.cuda_event for e in stage_events])
        code = load().ffn_sparse_forward_events(*args, arr)
    _check(code, "ffn_sparse_forward")
    return out


def ffn_sparse_gated_forward(x: torch.Tensor, w_gate_t: torch.Tensor, b_gate: torch.Tensor,
                             w_up_t: torch.Tensor, b_up: torch.Tensor, w_down: torch.Tensor,
                             tile: int, capacity: int, *, dense_capacity: Optional[int] = None,
                             out: Optional[ForwardBuffers] = None) -> ForwardBuffers:
    """y = (ReLU(x @ w_gate_t.T + b_gate) * (x @ w_up_t.T + b_up)) @ w_down with h
    in hybrid TwELL form (stored where the gate is non-zero).  Same buffers as
    ffn_sparse_forward (no debug h)."""
    dev = x.device
    n, dm = x.shape
    dff = w_gate_t.shape[0]
    dt = x.dtype
    _need(x, "x", dev, dt)
    for name, w in (("w_gate_t", w_gate_t), ("w_up_t", w_up_t), ("w_down", w_down)):
        _need(w, name, dev, dt, (dff, dm))
    _need(b_gate, "b_gate", dev, torch.float32, (dff,))
    _need(b_up, "b_up", dev, torch.float32, (dff,))
    if out is None:
        out = forward_buffers(n, dm, dff, tile, capacity, dt, dev, dense_capacity)
    shape = make_shape(n, dm, dff, tile, capacity, dt)
    _need(out.y, "y", dev, dt, (n, dm))
    out.hybrid.validate(dev)
    hs = out.hybrid.struct()
    _check(load().ffn_sparse_gated_forward(
        ctypes.byref(shape), _ptr(x), _ptr(w_gate_t), _ptr(b_gate), _ptr(w_up_t), _ptr(b_up),
        _ptr(w_down), _ptr(out.y), ctypes.byref(hs), _ptr(out.workspace), out.workspace.numel(),
        _ptr(out.status), _stream(dev)), "ffn_sparse_gated_forward")
    return out


def twell_pack(h: torch.Tensor, tile: int, capacity: int, *,
               dense_capacity: Optional[int] = None, out: Optional[Hybrid] = None,
               workspace: Optional[torch.Tensor] = None,
               status: Optional[torch.Tensor] = None):
    """dense_to_twell of h [N, d_ff]; returns (hybrid, device status word)."""
    dev = h.device
    n, dff = h.shape
    _need(h, "h", dev)
    shape = make_shape(n, 8, dff, tile, capacity, h.dtype)
    if out is None:
        out = Hybrid.empty(n, dff, tile, capacity, h.dtype, dev, dense_capacity)
    out.validate(dev)
    if workspace is None:
        workspace = torch.empty((max(pack_workspace_bytes(shape), 1),), dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=dev)
    hs = out.struct()
    code = load().twell_pack(ctypes.byref(shape), _ptr(h), ctypes.byref(hs), _ptr(workspace),
                             workspace.numel(), _ptr(status), _stream(dev))
    _check(code, "twell_pack")
    return out, status


def twell_pack_noalloc(h: torch.Tensor, tile: int, capacity: int, *,
                       dense_capacity: Optional[int] = None, out: Optional[Hybrid] = None,
                       status: Optional[torch.Tensor] = None):
    """dense_to_twell of h [N, d_ff] through the entry point that takes no
    workspace and allocates nothing (the library's fixed device scratch array
    stands in for it); returns (hybrid, device status word).  Outputs not
    passed in are allocated here, by PyTorch, before the call."""
    dev = h.device
    n, dff = h.shape
    _need(h, "h", dev)
    shape = make_shape(n, 8, dff, tile, capacity, h.dtype)
    if out is None:
        out = Hybrid.empty(n, dff, tile, capacity, h.dtype, dev, dense_capacity)
    out.validate(dev)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=dev)
    hs = out.struct()
    code = load().twell_pack_noalloc(ctypes.byref(shape), _ptr(h), ctypes.byref(hs), _ptr(status),
                                     _stream(dev))
    _check(code, "twell_pack_noalloc")
    return out, status


def twell_unpack(hy: Hybrid, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """twell_to_dense: the dense h [N, d_ff] of a hybrid."""
    dev = hy.values.device
    hy.validate(dev)
    if out is None:
        out = torch.empty((hy.n_rows, hy.d_ff), dtype=hy.dtype, device=dev)
    _need(out, "h", dev, hy.dtype, (hy.n_rows, hy.d_ff))
    shape = make_shape(hy.n_rows, 8, hy.d_ff, hy.tile, hy.capacity, hy.dtype)
    hs = hy.struct()
    _check(load().twell_unpack(ctypes.byref(shape), ctypes.byref(hs), _ptr(out), _stream(dev)),
           "twell_unpack")
    return out


def twell_spmm(hy: Hybrid, w_down: torch.Tensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, use_workspace: bool = True
               ) -> torch.Tensor:
    """The hybrid down-projection y [N, d_model] = unpack(hy) @ w_down.

    With `use_workspace` (the default) the dense rows' product splits K over
    a scratch buffer of twell_spmm_workspace_size bytes: `workspace` when
    given, else one allocated here; without it the library gets none."""
    dev = hy.values.device
    hy.validate(dev)
    dff, dm = w_down.shape
    _need(w_down, "w_down", dev, hy.dtype, (hy.d_ff, dm))
    if out is None:
        out = torch.empty((hy.n_rows, dm), dtype=hy.dtype, device=dev)
    _need(out, "y", dev, hy.dtype, (hy.n_rows, dm))
    shape = make_shape(hy.n_rows, dm, hy.d_ff, hy.tile, hy.capacity, hy.dtype)
    lib = load()
    ws_ptr, ws_bytes = None, 0
    if use_workspace:
        need = lib.twell_spmm_workspace_size(ctypes.byref(shape))
        if workspace is None and need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
        if workspace is not None:
            _need(workspace, "workspace", dev, torch.uint8)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    hs = hy.struct()
    _check(lib.twell_spmm(ctypes.byref(shape), ctypes.byref(hs), _ptr(w_down), _ptr(out), ws_ptr,
                          ws_bytes, _stream(dev)), "twell_spmm")
    return out


def spmm_workspace_bytes(shape: "Shape") -> int:
    """twell_spmm_workspace_size: bytes of twell_spmm's optional workspace."""
    return int(load().twell_spmm_workspace_size(ctypes.byref(shape)))


# ------------------------------------------------------------------ ELL rows
@dataclasses.dataclass
class Ell:
    """Device tensors of ELL rows (see twell_ell in twell.h): the non-zeros of
    each row in column order in the first counts[n] of `width` slots."""

    width: int
    d_ff: int
    values: torch.Tensor        # [N, width] dtype
    columns: torch.Tensor       # [N, width] uint16 bits (torch.int16)
    counts: torch.Tensor        # [N] uint16 bits (torch.int16)
    dense_rows: torch.Tensor    # [dense_capacity] int32
    dense_values: torch.Tensor  # [dense_capacity, d_ff] dtype
    n_dense: torch.Tensor       # [1] int32

    @property
    def n_rows(self) -> int:
        return self.counts.shape[0]

    @property
    def dense_capacity(self) -> int:
        return self.dense_rows.shape[0]

    @property
    def dtype(self) -> torch.dtype:
        return self.values.dtype

    @classmethod
    def empty(cls, n_rows: int, d_ff: int, width: int, dtype: torch.dtype, device,
              dense_capacity: Optional[int] = None) -> "Ell":
        cap = n_rows if dense_capacity is None else dense_capacity
        return cls(width, d_ff,
                   torch.empty((n_rows, width), dtype=dtype, device=device),
                   torch.empty((n_rows, width), dtype=torch.int16, device=device),
                   torch.empty((n_rows,), dtype=torch.int16, device=device),
                   torch.empty((cap,), dtype=torch.int32, device=device),
                   torch.empty((cap, d_ff), dtype=dtype, device=device),
                   torch.empty((1,), dtype=torch.int32, device=device))

    def struct(self) -> EllStruct:
        return EllStruct(_ptr(self.values), _ptr(self.columns), _ptr(self.counts),
                         _ptr(self.dense_rows), _ptr(self.dense_values), _ptr(self.n_dense),
                         self.dense_capacity)

    def validate(self, device) -> None:
        n, w = self.n_rows, self.width
        _need(self.values, "values", device, shape=(n, w))
        _need(self.columns, "columns", device, torch.int16, (n, w))
        _need(self.counts, "counts", device, torch.int16, (n,))
        _need(self.dense_rows, "dense_rows", device, torch.int32)
        _need(self.dense_values, "dense_values", device, self.values.dtype,
              (self.dense_capacity, self.d_ff))
        _need(self.n_dense, "n_dense", device, torch.int32, (1,))

    def n_dense_host(self) -> int:
        return int(self.n_dense.item())


def ell_shape(n_rows: int, d_model: int, d_ff: int, width: int, dtype: torch.dtype) -> Shape:
    """ELL rows are TwELL with one tile spanning the row: tile = d_ff, capacity = width."""
    return make_shape(n_rows, d_model, d_ff, d_ff, width, dtype)


def ell_pack(h: torch.Tensor, width: int, *, dense_capacity: Optional[int] = None,
             out: Optional[Ell] = None, workspace: Optional[torch.Tensor] = None,
             status: Optional[torch.Tensor] = None):
    """dense_to_ell of h [N, d_ff]; returns (ell, device status word)."""
    dev = h.device
    n, dff = h.shape
    _need(h, "h", dev)
    shape = ell_shape(n, 8, dff, width, h.dtype)
    if out is None:
        out = Ell.empty(n, dff, width, h.dtype, dev, dense_capacity)
    out.validate(dev)
    if workspace is None:
        ws = int(load().ell_pack_workspace_size(ctypes.byref(shape)))
        if ws == 0:
            raise TwellError(TWELL_ERR_INVALID_ARG, "ell_pack_workspace_size")
        workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=dev)
    es = out.struct()
    code = load().ell_pack(ctypes.byref(shape), _ptr(h), ctypes.byref(es), _ptr(workspace),
                           workspace.numel(), _ptr(status), _stream(dev))
    _check(code, "ell_pack")
    return out, status


def ell_unpack(e: Ell, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ell_to_dense: the dense h [N, d_ff] of ELL rows."""
    dev = e.values.device
    e.validate(dev)
    if out is None:
        out = torch.empty((e.n_rows, e.d_ff), dtype=e.dtype, device=dev)
    _need(out, "h", dev, e.dtype, (e.n_rows, e.d_ff))
    shape = ell_shape(e.n_rows, 8, e.d_ff, e.width, e.dtype)
    es = e.struct()
    _check(load().ell_unpack(ctypes.byref(shape), ctypes.byref(es), _ptr(out), _stream(dev)),
           "ell_unpack")
    return out


def ell_spmm(e: Ell, w_down: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The ELL down-projection y [N, d_model] = ell_to_dense(e) @ w_down."""
    dev = e.values.device
    e.validate(dev)
    dff, dm = w_down.shape
    _need(w_down, "w_down", dev, e.dtype, (e.d_ff, dm))
    if out is None:
        out = torch.empty((e.n_rows, dm), dtype=e.dtype, device=dev)
    _need(out, "y", dev, e.dtype, (e.n_rows, dm))
    shape = ell_shape(e.n_rows, dm, e.d_ff, e.width, e.dtype)
    es = e.struct()
    _check(load().ell_spmm(ctypes.byref(shape), ctypes.byref(es), _ptr(w_down), _ptr(out),
                           _stream(dev)), "ell_spmm")
    return out


# ------------------------------------------------------------------ backward
def backward_workspace_bytes(shape: Shape, dense_capacity: int) -> int:
    return int(load().ffn_sparse_backward_workspace_size(ctypes.byref(shape), dense_capacity))


@dataclasses.dataclass
class Grads:
    """Everything ffn_sparse_backward writes."""

    dx: torch.Tensor       # [N, d_model] dtype
    dw_up_t: torch.Tensor  # [d_ff, d_model] float32
    db_up: torch.Tensor    # [d_ff] float32
    dw_down: torch.Tensor  # [d_ff, d_model] float32


def ffn_sparse_backward(x: torch.Tensor, w_up_t: torch.Tensor, w_down: torch.Tensor,
                        hy: Hybrid, dy: torch.Tensor, *, out: Optional[Grads] = None,
                        workspace: Optional[torch.Tensor] = None) -> Grads:
    """Gradients of sum(y * dy) for y = ReLU(x @ w_up_t.T + b_up) @ w_down from
    the stored hybrid h of the forward pass: dx, dW_up^T, db_up, dW_down.

    x, dy [N, d_model]; w_up_t, w_down [d_ff, d_model]; all in h's dtype.
    Weight and bias gradients are float32.  Asynchronous like the forward."""
    dev = x.device
    n, dm = x.shape
    dt = x.dtype
    hy.validate(dev)
    _need(x, "x", dev, hy.dtype, (hy.n_rows, dm))
    _need(dy, "dy", dev, dt, (n, dm))
    _need(w_up_t, "w_up_t", dev, dt, (hy.d_ff, dm))
    _need(w_down, "w_down", dev, dt, (hy.d_ff, dm))
    shape = make_shape(n, dm, hy.d_ff, hy.tile, hy.capacity, dt)
    if out is None:
        out = Grads(torch.empty((n, dm), dtype=dt, device=dev),
                    torch.empty((hy.d_ff, dm), dtype=torch.float32, device=dev),
                    torch.empty((hy.d_ff,), dtype=torch.float32, device=dev),
                    torch.empty((hy.d_ff, dm), dtype=torch.float32, device=dev))
    _need(out.dx, "dx", dev, dt, (n, dm))
    _need(out.dw_up_t, "dw_up_t", dev, torch.float32, (hy.d_ff, dm))
    _need(out.db_up, "db_up", dev, torch.float32, (hy.d_ff,))
    _need(out.dw_down, "dw_down", dev, torch.float32, (hy.d_ff, dm))
    if workspace is None:
        ws = backward_workspace_bytes(shape, hy.dense_capacity)
        if ws == 0:
            raise TwellError(TWELL_ERR_UNSUPPORTED, "ffn_sparse_backward_workspace_size")
        workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
    hs = hy.struct()
    code = load().ffn_sparse_backward(
        ctypes.byref(shape), _ptr(x), _ptr(w_up_t), _ptr(w_down), ctypes.byref(hs), _ptr(dy),
        _ptr(out.dx), _ptr(out.dw_up_t), _ptr(out.db_up), _ptr(out.dw_down), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check(code, "ffn_sparse_backward")
    return out

