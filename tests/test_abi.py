"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and answers the host-only calls (version, status strings,
workspace sizes, argument validation) without touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from activation_sparse_transformer_amd import twell

# Tests that hand the library fake (never dereferenced) device addresses run
# only where no GPU could execute a kernel, should a host check ever miss.
no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake device pointers are passed only on a GPU-less host")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twell.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(twell.LIB_PATH):
        pytest.fail("libtwell.so is not built: run python -m activation_sparse_transformer_amd.build")
    return twell.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(twell.EXPORTS), names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", twell.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else of the library's own leaks out of the ABI
    ours = {n for n in exported if n.startswith(("twell", "ffn_", "ell_"))}
    assert ours == set(twell.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.twell_version() == 1
    assert twell.status_string(0) == "ok"
    assert "dense_capacity" in twell.status_string(twell.TWELL_ERR_DENSE_CAPACITY)
    assert twell.status_string(12345) == "unknown status"


def partials_d(rows_bucket, cols):
    return 32 * rows_bucket * cols * 4


def test_workspace_sizes(lib):
    s = twell.make_shape(4096, 2048, 8192, 128, 4, __import__("torch").bfloat16)
    ws = twell.ffn_workspace_bytes(s)
    # flags [N, nt] + row flags [N] + row map, sparse rows [N] int32 + a counter
    # (+ spill [N, d_ff] bf16 for the forward), each part 256-byte aligned
    route = 4096 * 64 + 4096 + 2 * 4096 * 4 + 256
    assert twell.pack_workspace_bytes(s) == route
    assert ws == route + 4096 * 8192 * 2
    # at most 64 rows: split-K partial sums too, fp32 [up to 32 K slices][16/32/64 rows]
    # [the wider of d_ff and d_model]
    d = twell.make_shape(16, 4096, 16384, 128, 4, __import__("torch").bfloat16)
    pack = 2048 + 256 + 2 * 256 + 256
    spill = 16 * 16384 * 2
    partials = 32 * 16 * 16384 * 4
    assert twell.pack_workspace_bytes(d) == pack
    assert twell.ffn_workspace_bytes(d) == pack + spill + partials
    t = twell.make_shape(40, 136, 768, 128, 4, __import__("torch").bfloat16)  # 32 < 40 <= 64 rows
    partials = 32 * 64 * 768 * 4
    assert twell.ffn_workspace_bytes(t) == twell.pack_workspace_bytes(t) + 40 * 768 * 2 + partials
    # twell_spmm's optional workspace: the split-K partial sums of at most 64
    # rows (as the forward's), else bf16 32 K slices of every row, at most 32 MiB
    assert twell.spmm_workspace_bytes(d) == partials_d(16, 16384)
    assert twell.spmm_workspace_bytes(t) == 32 * 64 * 768 * 4
    assert twell.spmm_workspace_bytes(s) == 32 << 20
    small = twell.make_shape(333, 256, 1024, 128, 4, __import__("torch").bfloat16)
    assert twell.spmm_workspace_bytes(small) == 32 * 333 * 256 * 4
    f32 = twell.make_shape(300, 256, 1024, 128, 4, __import__("torch").float32)
    assert twell.spmm_workspace_bytes(f32) == 0
    bad = twell.make_shape(16, 2048, 8192, 100, 4, __import__("torch").bfloat16)
    assert twell.ffn_workspace_bytes(bad) == 0


def _call_forward(lib, shape, hybrid):
    return lib.ffn_sparse_forward(ctypes.byref(shape), None, None, None, None, None,
                                  ctypes.byref(hybrid) if hybrid is not None else None,
                                  None, None, 0, None, None)


@no_gpu_only
@pytest.mark.parametrize("field,value,code", [
    ("tile", 100, twell.TWELL_ERR_INVALID_ARG),      # does not divide d_ff
    ("tile", 32, twell.TWELL_ERR_UNSUPPORTED),       # valid geometry, no kernel
    ("capacity", 0, twell.TWELL_ERR_INVALID_ARG),
    ("capacity", 129, twell.TWELL_ERR_INVALID_ARG),  # > T
    ("d_model", 12, twell.TWELL_ERR_INVALID_ARG),    # not a multiple of 8
    ("n_rows", -1, twell.TWELL_ERR_INVALID_ARG),
    ("dtype", 7, twell.TWELL_ERR_INVALID_ARG),
    ("reserved", 1, twell.TWELL_ERR_INVALID_ARG),
])
def test_shape_validation(lib, field, value, code):
    s = twell.Shape(64, 128, 512, 128, 4, 1, 0)
    setattr(s, field, value)
    h = twell.HybridStruct(1, 1, 1, None, None, 1, 0)
    assert _call_forward(lib, s, h) == code


@no_gpu_only
def test_null_arguments_rejected_on_host(lib):
    s = twell.Shape(64, 128, 512, 128, 4, 1, 0)
    assert _call_forward(lib, s, None) == twell.TWELL_ERR_INVALID_ARG
    h = twell.HybridStruct(1, 1, 1, None, None, 1, 0)
    assert _call_forward(lib, s, h) == twell.TWELL_ERR_INVALID_ARG  # x etc. are NULL
    h_nodense = twell.HybridStruct(1, 1, 1, None, None, 1, 5)  # capacity 5, no buffers
    assert lib.twell_unpack(ctypes.byref(s), ctypes.byref(h_nodense), 1, None) == \
        twell.TWELL_ERR_INVALID_ARG
    assert lib.twell_spmm(None, ctypes.byref(h), 1, 1, None, 0, None) == \
        twell.TWELL_ERR_INVALID_ARG


@no_gpu_only
def test_workspace_too_small_rejected_on_host(lib):
    s = twell.Shape(64, 128, 512, 128, 4, 1, 0)
    a = 4096  # a well-aligned address that the host-side checks never dereference
    h = twell.HybridStruct(a, a, a, None, None, a, 0)
    rc = lib.ffn_sparse_forward(ctypes.byref(s), a, a, a, a, a, ctypes.byref(h), None, a, 16,
                                None, None)
    assert rc == twell.TWELL_ERR_WORKSPACE
    rc = lib.twell_pack(ctypes.byref(s), a, ctypes.byref(h), a, 16, None, None)
    assert rc == twell.TWELL_ERR_WORKSPACE
    # twell_spmm: no workspace is fine; a given one must be large enough
    need = lib.twell_spmm_workspace_size(ctypes.byref(s))
    assert need > 16
    rc = lib.twell_spmm(ctypes.byref(s), ctypes.byref(h), a, a, a, 16, None)
    assert rc == twell.TWELL_ERR_WORKSPACE
    rc = lib.twell_spmm(ctypes.byref(s), ctypes.byref(h), a, a, a + 8, need, None)
    assert rc == twell.TWELL_ERR_INVALID_ARG
    # a misaligned pointer is rejected before the size check
    rc = lib.twell_pack(ctypes.byref(s), a + 2, ctypes.byref(h), a, 1 << 30, None, None)
    assert rc == twell.TWELL_ERR_INVALID_ARG


@no_gpu_only
def test_noalloc_pack_rejects_shapes_beyond_its_scratch(lib):
    # 262144 rows x 64 tiles of flags alone is 16 MiB: past the fixed scratch
    s = twell.Shape(262144, 8, 64 * 128, 128, 4, 1, 0)
    assert lib.twell_pack_workspace_size(ctypes.byref(s)) > twell.NOALLOC_SCRATCH_BYTES
    a = 4096
    h = twell.HybridStruct(a, a, a, None, None, a, 0)
    assert lib.twell_pack_noalloc(ctypes.byref(s), a, ctypes.byref(h), None, None) == \
        twell.TWELL_ERR_SCRATCH_LIMIT
    assert "scratch" in twell.status_string(twell.TWELL_ERR_SCRATCH_LIMIT)


def _align(v):
    return (v + 255) // 256 * 256


def test_backward_workspace_size(lib):
    """The (neuron, row) bitmap and one row flag per token, dz in h's slots
    and dense rows, the bitmap's word prefixes, per-neuron counts and offsets,
    one 16-byte entry per slot and per stored dense element, and (at most 64
    rows) the fallback's split-K partial sums; each part 256-byte aligned."""
    n, dm, dff, T, C, cap = 4096, 2048, 8192, 128, 4, 512
    s = twell.make_shape(n, dm, dff, T, C, torch.bfloat16)
    slots = n * (dff // T) * C
    words = dff * ((n + 63) // 64)
    ents = slots + cap * dff
    want = (_align(words * 8) + _align(n) + _align(slots * 2) + _align(cap * dff * 2) +
            _align(words * 4) + _align(dff * 4) + _align((dff + 1) * 4) + _align(ents * 16) +
            _align(8 * ents * 4))  # partial dots of dz, one per column slice (8 XCDs)
    assert twell.backward_workspace_bytes(s, cap) == want
    # dense capacity past n_rows counts as n_rows
    assert twell.backward_workspace_bytes(s, 10 * n) == twell.backward_workspace_bytes(s, n)
    # 40 rows: the fallback's split-K partial sums fp32 [32 slices][64 rows][768]
    small = twell.make_shape(40, 136, 768, 128, 4, torch.bfloat16)
    slots, words = 40 * 6 * 4, 768
    want = (_align(words * 8) + _align(40) + _align(slots * 2) + _align(words * 4) +
            _align(768 * 4) + _align(769 * 4) + _align(slots * 16) + _align(slots * 4) +
            32 * 64 * 768 * 4)  # d_model 136 is one column slice
    assert twell.backward_workspace_bytes(small, 0) == want
    # invalid: negative capacity, a bad shape, more entries than an int32 can place
    assert twell.backward_workspace_bytes(s, -1) == 0
    assert twell.backward_workspace_bytes(twell.make_shape(16, 2048, 8192, 100, 4,
                                                          torch.bfloat16), 0) == 0
    huge = twell.make_shape(1 << 20, 8, 65536, 256, 255, torch.bfloat16)  # 2^20 * 256 * 255 slots
    assert twell.backward_workspace_bytes(huge, 0) == 0


@no_gpu_only
def test_backward_host_checks(lib):
    s = twell.Shape(64, 128, 512, 128, 4, 1, 0)
    a = 4096
    h = twell.HybridStruct(a, a, a, None, None, a, 0)
    ws = lib.ffn_sparse_backward_workspace_size(ctypes.byref(s), 0)
    call = lambda **kw: lib.ffn_sparse_backward(
        ctypes.byref(s), kw.get("x", a), a, a, ctypes.byref(h), a, kw.get("dx", a),
        kw.get("dwu", a), a, a, kw.get("ws", a), kw.get("wsb", ws), None)
    assert call(wsb=ws - 1) == twell.TWELL_ERR_WORKSPACE
    assert call(ws=None) == twell.TWELL_ERR_INVALID_ARG
    assert call(dwu=None) == twell.TWELL_ERR_INVALID_ARG
    assert call(x=None) == twell.TWELL_ERR_INVALID_ARG
    assert call(dx=a + 4) == twell.TWELL_ERR_INVALID_ARG  # misaligned
    bad = twell.HybridStruct(a, a, a, None, None, a, -1)
    assert lib.ffn_sparse_backward(ctypes.byref(s), a, a, a, ctypes.byref(bad), a, a, a, a, a, a,
                                   ws, None) == twell.TWELL_ERR_INVALID_ARG
