"""GPU parity of every C-ABI entry point against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.

Bars: TwELL packing bit-exact (indices, counts, values as bit patterns, dense
row list, dense rows); y and h within max|err| <= tol * max|ref| with tol =
1e-4 (float32) / 1e-2 (bfloat16); integer-valued products exact.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_transformer_amd import twell
from activation_sparse_transformer_amd.synth import CONFIGS, make_inputs
from gpu_helpers import (TOL, as_f32, as_f64, assert_close_rel, assert_pack_matches,
                         inputs_to_device, oracle_inputs, say, u32)

pytestmark = pytest.mark.gpu
DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def sparse_h(seed, n, dff, density, dtype, negzero=False, nan=False):
    rng = np.random.default_rng(seed)
    h = np.abs(rng.standard_normal((n, dff))).astype(np.float32) + 0.01
    h *= np.where(rng.random((n, dff)) < 0.5, 1, -1).astype(np.float32)
    h[rng.random((n, dff)) >= density] = 0.0
    if negzero:
        h[(h == 0) & (rng.random((n, dff)) < 0.3)] = -0.0
    if nan and n:
        h[rng.integers(0, n, 3), rng.integers(0, dff, 3)] = np.nan
    t = torch.from_numpy(h).to(dtype)
    return t, as_f32(t)  # GPU input and its exact float32 value on the host


# ---------------------------------------------------------------- pack / unpack
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("T,C,density", [(64, 8, 0.08), (128, 4, 0.02), (256, 8, 0.03), (128, 1, 0.005)])
@pytest.mark.parametrize("n", [1, 77, 300])
def test_pack_unpack_bitexact(dtype, T, C, density, n):
    say(f"pack/unpack {dtype} T={T} C={C} n={n}")
    dff = T * 5
    ht, hh = sparse_h(1000 + T + C + n, n, dff, density, DT[dtype], negzero=True, nan=(n == 300))
    hy, status = twell.twell_pack(ht.cuda(), T, C)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_OK
    ref = assert_pack_matches(hy, hh)
    u = twell.twell_unpack(hy)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(as_f32(u)), u32(oracle.unpack(ref)))


@pytest.mark.parametrize("n,dff,T,density", [(64, 1024, 64, 0.03), (65, 1024, 64, 0.03),
                                             (1024, 1024, 64, 0.02), (1000, 192, 64, 0.06),
                                             (1025, 1024, 64, 0.02), (2500, 200 * 64, 64, 0.01),
                                             (16384, 512, 128, 0.01), (16385, 512, 128, 0.01)])
def test_pack_routing_row_counts(n, dff, T, density):
    """Row routing on both sides of every switch: inside the dense-row build's
    workgroups (up to 64 rows), the scan with the row flags ORed inside it (up
    to 1024), the build counting dense rows below each row after the row pass
    (up to 16384), the row pass and the scan beyond; tile counts a multiple
    of 16 or not."""
    say(f"pack routing n={n} dff={dff} T={T}")
    ht, hh = sparse_h(77 + n, n, dff, density, torch.bfloat16)
    hy, status = twell.twell_pack(ht.cuda(), T, 4)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_OK
    ref = assert_pack_matches(hy, hh)
    assert 0 < ref.n_dense < n


def test_pack_all_zero_and_all_dense():
    for fill, dense in ((0.0, False), (1.5, True)):
        h = torch.full((40, 512), fill, dtype=torch.bfloat16, device="cuda")
        hy, status = twell.twell_pack(h, 128, 4)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert hy.n_dense_host() == (40 if dense else 0)
        assert_pack_matches(hy, as_f32(h))


def test_pack_dense_capacity_exceeded():
    ht, hh = sparse_h(5, 200, 512, 0.06, torch.bfloat16)
    ref = oracle.pack(hh, 128, 4)
    assert ref.n_dense > 10
    hy, status = twell.twell_pack(ht.cuda(), 128, 4, dense_capacity=10)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_ERR_DENSE_CAPACITY
    assert hy.n_dense_host() == ref.n_dense
    np.testing.assert_array_equal(hy.dense_rows.cpu().numpy(), ref.dense_rows[:10])
    np.testing.assert_array_equal(u32(as_f32(hy.dense_values)), u32(ref.dense_values[:10]))
    # every dense row, stored or not, has cleared TwELL slots
    np.testing.assert_array_equal(hy.counts.cpu().numpy(), ref.counts)
    np.testing.assert_array_equal(u32(as_f32(hy.values)), u32(ref.values))


@pytest.mark.parametrize("dtype,dff", [("fp32", 16384), ("bf16", 32768)])
def test_pack_long_rows_two_pass(dtype, dff):
    """Rows of 64 KB: the dense rows are copied straight from h, with no row
    buffer in LDS."""
    say(f"pack long rows {dtype} dff={dff}")
    ht, hh = sparse_h(31, 37, dff, 0.01, DT[dtype])
    hy, status = twell.twell_pack(ht.cuda(), 256, 8)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_OK
    ref = assert_pack_matches(hy, hh)
    assert 0 < ref.n_dense < 37
    u = twell.twell_unpack(hy)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(as_f32(u)), u32(oracle.unpack(ref)))


def test_pack_zero_rows():
    h = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    hy, status = twell.twell_pack(h, 128, 4)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and hy.n_dense_host() == 0
    assert twell.twell_unpack(hy).shape == (0, 256)


# ------------------------------------------------------------------------ spmm
@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,dm,T,C", [(50, 136, 64, 4), (300, 520, 128, 4), (130, 64, 256, 8),
                                      (70, 2048, 128, 4), (33, 4096, 64, 2), (20, 8192, 256, 8)])
def test_spmm_integer_exact(dtype, n, dm, T, C, use_ws):
    """With and without twell_spmm's workspace (the dense rows' K split over
    workgroups into partial sums, or one workgroup per output tile)."""
    say(f"spmm integer {dtype} n={n} dm={dm} T={T} workspace={use_ws}")
    rng = np.random.default_rng(n + dm)
    dff = 3 * T
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) < 0.96] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.7] = 0
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(DT[dtype]).cuda(), T, C)
    y = twell.twell_spmm(hy, torch.from_numpy(w).to(DT[dtype]).cuda(), use_workspace=use_ws)
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert ref_h.n_dense > 0 and ref_h.n_dense < n
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    assert np.max(np.abs(y_ref)) <= 256  # every value and partial sum is exact in bf16 / fp32
    np.testing.assert_array_equal(as_f64(y), y_ref)


@pytest.mark.parametrize("n,dm,dff,T,density", [
    (4500, 512, 512, 128, 0.01),  # many row batches per wave of the XCD-sliced kernel
    (400, 40, 9728, 128, 0.01),   # a long d_ff with a d_model the sliced kernel does not take
    (128, 1024, 896, 64, 0.03),   # d_model of two XCD slices
])
def test_spmm_many_rows_integer_exact(n, dm, dff, T, density):
    """Every row checked, with values whose products and sums are exact."""
    say(f"spmm rows n={n} dm={dm} dff={dff} T={T}")
    rng = np.random.default_rng(n + dff)
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= density] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.7] = 0
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(torch.bfloat16).cuda(), T, 4)
    y = twell.twell_spmm(hy, torch.from_numpy(w).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert 0 < ref_h.n_dense < n
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    assert np.max(np.abs(y_ref)) <= 256
    np.testing.assert_array_equal(as_f64(y), y_ref)


@pytest.mark.parametrize("n,dm,dff,C", [(1500, 512, 4096, 4), (1500, 1024, 8192, 4),
                                         (1300, 512, 8192, 8)])
def test_spmm_whole_wave_rows_integer_exact(n, dm, dff, C):
    """Rows whose slots fill whole waves (2, 4 or 8 slots per lane): each lane
    loads its slots in one round; every value of y checked, exact."""
    T = 128
    say(f"spmm whole-wave rows n={n} dm={dm} dff={dff} C={C}")
    rng = np.random.default_rng(n + dff + C)
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= (0.01 if C == 4 else 0.03)] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.7] = 0
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(torch.bfloat16).cuda(), T, C)
    y = twell.twell_spmm(hy, torch.from_numpy(w).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert 0 < ref_h.n_dense < n
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    assert np.max(np.abs(y_ref)) <= 256
    np.testing.assert_array_equal(as_f64(y), y_ref)


@pytest.mark.parametrize("n,dm,dff,rate", [(16, 4096, 16384, 0.008), (4096, 2048, 8192, 0.011),
                                            (4096, 2048, 8192, 0.006)])
def test_spmm_workspace_split_integer_exact(n, dm, dff, rate):
    """twell_spmm with its workspace on the decode and 1B shapes: few and many
    dense rows, so the fallback's K split ranges from 2 to 32 slices (and the
    split-K kernels of at most 64 rows); y the same as without the workspace
    and as the oracle, exactly (integer values)."""
    say(f"spmm workspace split n={n} dm={dm} dff={dff} rate={rate}")
    T, C = 128, 4
    rng = np.random.default_rng(n + dff + int(rate * 1000))
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= rate] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.9] = 0
    wd = torch.from_numpy(w).to(torch.bfloat16).cuda()
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(torch.bfloat16).cuda(), T, C)
    y = twell.twell_spmm(hy, wd)
    y0 = twell.twell_spmm(hy, wd, use_workspace=False)
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert 0 < ref_h.n_dense < n
    np.testing.assert_array_equal(u32(as_f32(y)), u32(as_f32(y0)))
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    assert np.max(np.abs(y_ref)) <= 256  # every partial sum exact in fp32, the result in bf16
    np.testing.assert_array_equal(as_f64(y), y_ref)


def test_spmm_large_fallback_tiles_integer_exact():
    """Enough rows and columns for the fallback's 256 x 256 tiles (at least
    2048 of them in the worst case): about half of 8000 rows dense, every
    value of y checked, all products and sums exact in bf16."""
    n, dm, T = 8000, 16384, 128
    say(f"spmm large fallback tiles n={n} dm={dm}")
    rng = np.random.default_rng(8000)
    h = rng.integers(-2, 3, size=(n, T)).astype(np.float32)
    h[rng.random((n, T)) >= 0.013] = 0
    w = rng.integers(-1, 2, size=(T, dm)).astype(np.float32)
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(torch.bfloat16).cuda(), T, 1)
    y = twell.twell_spmm(hy, torch.from_numpy(w).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert n // 4 < ref_h.n_dense < 3 * n // 4
    y_ref = (oracle.unpack(ref_h) @ w).astype(np.float32)  # integers below 2^8: exact
    assert np.max(np.abs(y_ref)) <= 256
    np.testing.assert_array_equal(as_f32(y), y_ref)


@pytest.mark.parametrize("dtype,n,dm", [("fp32", 1200, 512), ("bf16", 1500, 136)])
def test_spmm_wave_per_chunk_integer_exact(dtype, n, dm):
    """Enough (row, 64-lane column chunk) pairs (more than 1024) that the
    sparse product runs one wave per pair: float32 at any width, bf16 at a
    d_model the XCD-sliced kernel does not take.  Every value of y checked,
    all products and sums exact."""
    say(f"spmm wave-per-chunk {dtype} n={n} dm={dm}")
    rng = np.random.default_rng(n + dm + 7)
    T, C, dff = 128, 4, 1024
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= 0.012] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.7] = 0
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(DT[dtype]).cuda(), T, C)
    y = twell.twell_spmm(hy, torch.from_numpy(w).to(DT[dtype]).cuda())
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert 0 < ref_h.n_dense < n
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    assert np.max(np.abs(y_ref)) <= 256
    np.testing.assert_array_equal(as_f64(y), y_ref)


@pytest.mark.parametrize("dtype,n,dm", [("bf16", 40, 1024), ("bf16", 3000, 2048),
                                        ("fp32", 50, 136), ("fp32", 1200, 512)])
def test_spmm_writes_each_row_once(dtype, n, dm):
    """twell_spmm writes every row of y once: the rows listed among the stored
    dense rows through the fallback only, every other row through the sparse
    kernel.  A NaN sentinel in y beforehand survives nowhere; then, with the
    stored dense rows overwritten by other values after the pack, the dense
    rows of y follow those values (the sparse kernel does not write them
    after, or instead of, the fallback)."""
    say(f"spmm each row once {dtype} n={n} dm={dm}")
    rng = np.random.default_rng(n * 3 + dm)
    T, C, dff = 128, 4, 512
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= 0.02] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    hy, _ = twell.twell_pack(torch.from_numpy(h).to(DT[dtype]).cuda(), T, C)
    torch.cuda.synchronize()
    ref_h = assert_pack_matches(hy, h)
    assert 0 < ref_h.n_dense < n
    wd = torch.from_numpy(w).to(DT[dtype]).cuda()
    y = torch.full((n, dm), float("nan"), dtype=DT[dtype], device="cuda")
    twell.twell_spmm(hy, wd, out=y)
    torch.cuda.synchronize()
    y_ref = oracle.spmm(ref_h, w.astype(np.float64))
    np.testing.assert_array_equal(as_f64(y), y_ref)  # no NaN sentinel survives
    # with the stored dense rows forged to hold other values, the dense rows
    # of y follow them: the sparse kernel wrote nothing there after the fallback
    nd = hy.n_dense_host()
    hy.dense_values[:nd] = 1
    twell.twell_spmm(hy, wd, out=y)
    torch.cuda.synchronize()
    forged = ref_h.values.copy(), ref_h.dense_values.copy()
    ref_h.dense_values[:] = 1
    y_ref2 = oracle.spmm(ref_h, w.astype(np.float64))
    ref_h.values, ref_h.dense_values = forged
    np.testing.assert_array_equal(as_f64(y), y_ref2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_spmm_identity_is_unpack(dtype):
    ht, hh = sparse_h(9, 90, 256, 0.05, DT[dtype])
    hy, _ = twell.twell_pack(ht.cuda(), 64, 4)
    eye = torch.eye(256, dtype=DT[dtype], device="cuda")
    y = twell.twell_spmm(hy, eye)
    u = twell.twell_unpack(hy)
    torch.cuda.synchronize()
    assert hy.n_dense_host() > 0
    np.testing.assert_array_equal(u32(as_f32(y)), u32(as_f32(u)))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_spmm_random_within_tolerance(dtype):
    ht, hh = sparse_h(11, 257, 640, 0.03, DT[dtype])
    rng = np.random.default_rng(2)
    w = torch.from_numpy(rng.standard_normal((640, 328)).astype(np.float32)).to(DT[dtype])
    hy, _ = twell.twell_pack(ht.cuda(), 128, 4)
    y = twell.twell_spmm(hy, w.cuda())
    torch.cuda.synchronize()
    ref = oracle.spmm(oracle.pack(hh, 128, 4), as_f64(w))
    assert_close_rel(as_f64(y), ref, TOL[DT[dtype]])


# --------------------------------------------------------------------- forward
SMALL = [
    # (config, n_rows, d_model, d_ff): ragged N, K tails, partial column blocks
    ("tiny_fp32", 64, 128, 512),
    ("tiny_fp32", 45, 72, 320),
    ("ffn_1b_bf16", 300, 200, 640),
    ("ffn_1b_bf16", 37, 256, 384),
    ("ffn_1b_bf16", 1, 64, 128),
    ("hybrid_stress_bf16", 260, 264, 1152),
    ("decode_bf16", 16, 512, 1024),
    ("large_bf16", 129, 136, 768),
    # K a multiple of 64 and >= 128 rows: the direct-to-LDS MFMA kernels,
    # with ragged row counts and partial column blocks
    ("ffn_1b_bf16", 300, 256, 640),
    ("hybrid_stress_bf16", 520, 512, 1536),
    ("large_bf16", 257, 192, 1280),
    ("decode_bf16", 16, 256, 512),
    # at most 64 rows: split-K partial sums (MFMA when d_model is a multiple of
    # 64, the general up-projection kernel otherwise), 33..64 rows on 64-row blocks
    ("decode_bf16", 16, 136, 1024),
    ("ffn_1b_bf16", 64, 576, 1280),
    ("decode_bf16", 3, 4096, 2048),
    # d_model/8 a whole 4, 8 or 16 bf16 per lane: the XCD-sliced sparse product
    ("ffn_1b_bf16", 150, 2048, 512),
    ("hybrid_stress_bf16", 40, 4096, 384),
    ("large_bf16", 24, 8192, 512),
    # a float32 row longer than 64 KB: dense rows rebuilt without the LDS row buffer
    ("tiny_fp32", 20, 64, 16448),
    # bf16 rows over 20 KB with 4 or 8 slots per tile: dense rows rebuilt from slot groups
    # (at most 64 rows: the build routes the rows itself)
    ("ffn_1b_bf16", 70, 128, 10368),
    ("large_bf16", 33, 64, 10752),
    ("ffn_1b_bf16", 64, 192, 10368),
    ("decode_bf16", 1, 128, 12288),
    # 65 rows: past the split-K kernels and the in-workgroup routing
    ("ffn_1b_bf16", 65, 192, 2048),
]


def run_forward(cfg, t, debug=True, dense_capacity=None):
    d = inputs_to_device(t)
    out = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                   cfg.capacity, dense_capacity=dense_capacity, debug_h=debug)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,n,dm,dff", SMALL)
def test_forward_small(name, n, dm, dff):
    cfg = CONFIGS[name].replace(n_rows=n, d_model=dm, d_ff=dff)
    say(f"forward {name} n={n} dm={dm} dff={dff}")
    t = make_inputs(cfg)
    out = run_forward(cfg, t)
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    tol = TOL[cfg.torch_dtype]
    assert_close_rel(as_f64(out.h_debug), h_ref, tol, "h")
    ref = assert_pack_matches(out.hybrid, as_f32(out.h_debug))
    assert_close_rel(as_f64(out.y), y_ref, tol, "y")
    say(f"  n_dense={ref.n_dense}")
    # the debug store changes nothing, and the pass is deterministic
    out2 = run_forward(cfg, t, debug=False)
    np.testing.assert_array_equal(u32(as_f32(out2.y)), u32(as_f32(out.y)))
    np.testing.assert_array_equal(out2.hybrid.counts.cpu().numpy(), out.hybrid.counts.cpu().numpy())
    np.testing.assert_array_equal(u32(as_f32(out2.hybrid.values)), u32(as_f32(out.hybrid.values)))


@pytest.mark.parametrize("n,dm,dff", [(300, 256, 1024), (1500, 512, 2048), (130, 136, 576)])
def test_forward_fp32_many_rows(n, dm, dff):
    """float32 batches of more than 64 rows: the VALU up-projection's pack with
    partially filled tiles (0 < count <= C and count > C both occur), the
    generic fallback and the float32 sparse kernels; pack bit-exact against
    the oracle's packer on the GPU's own h, h and y within 1e-4."""
    cfg = CONFIGS["tiny_fp32"].replace(n_rows=n, d_model=dm, d_ff=dff)
    say(f"forward fp32 n={n} dm={dm} dff={dff}")
    t = make_inputs(cfg)
    out = run_forward(cfg, t)
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    tol = TOL[cfg.torch_dtype]
    assert_close_rel(as_f64(out.h_debug), h_ref, tol, "h")
    ref = assert_pack_matches(out.hybrid, as_f32(out.h_debug))
    cnt = ref.counts
    assert np.any((cnt > 0) & (cnt <= cfg.capacity)) and 0 < ref.n_dense < n
    assert_close_rel(as_f64(out.y), y_ref, tol, "y")
    say(f"  n_dense={ref.n_dense}")


@pytest.mark.parametrize("n,dm,dff,C", [(300, 256, 1024, 4), (260, 128, 1280, 16), (130, 192, 768, 17),
                                         (129, 64, 576, 4)])
def test_forward_tile64_bf16(n, dm, dff, C):
    """bf16 with T = 64: the LDS pack epilogue with slots staged (C <= 8) or
    stored per thread (C = 16, up to 64 slots per block row); C = 17 takes
    the other epilogue; d_ff = 576 (9 tiles) leaves the last block's columns
    past d_ff unused.  Pack bit-exact, h and y within tolerance."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=n, d_model=dm, d_ff=dff, tile=64, capacity=C)
    say(f"forward bf16 T=64 n={n} dm={dm} dff={dff} C={C}")
    t = make_inputs(cfg)
    # ~4% active at C = 4, ~15% at C >= 16: tiles both fit and overflow
    t["b_up"] = t["b_up"] + (0.6 if C <= 4 else 1.6)
    out = run_forward(cfg, t)
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    tol = TOL[cfg.torch_dtype]
    assert_close_rel(as_f64(out.h_debug), h_ref, tol, "h")
    ref = assert_pack_matches(out.hybrid, as_f32(out.h_debug))
    assert 0 < ref.n_dense < n
    assert_close_rel(as_f64(out.y), y_ref, tol, "y")


@pytest.mark.parametrize("C", [5, 8, 16, 64, 128])
def test_forward_capacities(C):
    """The 1B layer's tile width with other capacities (the capacity sweep):
    staged and unstaged pack epilogues, slot lists in LDS or not, C = T."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=300, d_model=256, d_ff=1024, capacity=C)
    say(f"forward capacity {C}")
    t = make_inputs(cfg)
    t["b_up"] = t["b_up"] + 1.2  # ~10% active: some tiles overflow even at larger C
    out = run_forward(cfg, t)
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    tol = TOL[cfg.torch_dtype]
    assert_close_rel(as_f64(out.h_debug), h_ref, tol, "h")
    assert_pack_matches(out.hybrid, as_f32(out.h_debug))
    assert_close_rel(as_f64(out.y), y_ref, tol, "y")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_forward_bias_limits(dtype):
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=150, d_model=128, d_ff=512, dtype=dtype)
    t = make_inputs(cfg)
    t["b_up"] = torch.full_like(t["b_up"], -1e4)
    out = run_forward(cfg, t)
    assert out.hybrid.n_dense_host() == 0
    assert torch.all(out.hybrid.counts == 0)
    assert torch.all(out.y.view(torch.int16 if dtype == "bf16" else torch.int32) == 0)  # +0 bits
    t["b_up"] = torch.full_like(t["b_up"], 1e4)
    out = run_forward(cfg, t)
    assert out.hybrid.n_dense_host() == 150  # every tile is full, every row dense
    _, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    assert_close_rel(as_f64(out.y), y_ref, TOL[cfg.torch_dtype])


@pytest.mark.parametrize("n_rows,d_ff", [(200, 1024), (1500, 1024), (60, 2048), (48, 12288)])
def test_forward_dense_capacity_exceeded(n_rows, d_ff):
    """Too many dense rows: the status says so, n_dense is the true count and
    the first dense_capacity dense rows are stored, whether the capacity runs
    out early or at the last dense row, with the row flags ORed inside the
    scan (200 rows), by the separate row pass (1500 rows), or by the dense-row
    build itself (at most 64 rows: rows of 4 KB built in LDS, of 24 KB from
    slot groups)."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=n_rows, d_model=128, d_ff=d_ff)
    t = make_inputs(cfg)
    total = run_forward(cfg, t).hybrid.n_dense_host()
    for cap in (3, total - 1):
        out = run_forward(cfg, t, dense_capacity=cap)
        h_ref = oracle.pack(as_f32(out.h_debug), cfg.tile, cfg.capacity)
        assert h_ref.n_dense == total > cap
        assert int(out.status.item()) == twell.TWELL_ERR_DENSE_CAPACITY
        assert out.hybrid.n_dense_host() == total
        np.testing.assert_array_equal(out.hybrid.dense_rows.cpu().numpy(), h_ref.dense_rows[:cap])


def test_forward_zero_rows():
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=0, d_model=128, d_ff=512)
    t = make_inputs(cfg)
    out = run_forward(cfg, t)
    assert int(out.status.item()) == 0 and out.hybrid.n_dense_host() == 0
    assert out.y.shape == (0, 128)


def test_forward_matches_standalone_pack_and_spmm():
    """The fused path's hybrid equals pack(h) bit for bit, and its y equals
    twell_spmm of that hybrid bit for bit on the sparse rows; on the dense
    rows within tolerance (the two may split the fallback's K differently,
    with partial sums in different workspaces), both against the oracle."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=333, d_model=256, d_ff=1024)
    t = make_inputs(cfg)
    out = run_forward(cfg, t)
    hy, _ = twell.twell_pack(out.h_debug, cfg.tile, cfg.capacity)
    y2 = twell.twell_spmm(hy, t["w_down"].cuda())
    torch.cuda.synchronize()
    for a, b in ((out.hybrid.counts, hy.counts), (out.hybrid.indices, hy.indices)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    np.testing.assert_array_equal(u32(as_f32(out.hybrid.values)), u32(as_f32(hy.values)))
    nd = hy.n_dense_host()
    assert nd == out.hybrid.n_dense_host() and nd > 0
    np.testing.assert_array_equal(u32(as_f32(out.hybrid.dense_values[:nd])),
                                  u32(as_f32(hy.dense_values[:nd])))
    sparse = np.ones(cfg.n_rows, dtype=bool)
    sparse[hy.dense_rows[:nd].cpu().numpy()] = False
    np.testing.assert_array_equal(u32(as_f32(out.y))[sparse], u32(as_f32(y2))[sparse])
    _, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    assert_close_rel(as_f64(out.y), y_ref, TOL[cfg.torch_dtype], "forward y")
    assert_close_rel(as_f64(y2), y_ref, TOL[cfg.torch_dtype], "twell_spmm y")


def integer_layer(seed, n, dm, dff, b0):
    """A layer whose every intermediate is a small integer: x, W_up, W_down in
    {-1, 0, 1}, an integer bias.  z, h and y are then exact in bf16 storage
    and float32 accumulation in any order (|h| < 16, |y| < 64), so the
    forward's y must equal the oracle's bit for bit however it splits and
    orders its sums."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-1, 2, size=(n, dm)); x[rng.random((n, dm)) < 0.7] = 0
    wu = rng.integers(-1, 2, size=(dff, dm)); wu[rng.random((dff, dm)) < 0.7] = 0
    wd = rng.integers(-1, 2, size=(dff, dm)); wd[rng.random((dff, dm)) < 0.8] = 0
    b = np.full(dff, float(b0))
    t = {"x": torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16),
         "w_up_t": torch.from_numpy(wu.astype(np.float32)).to(torch.bfloat16),
         "b_up": torch.from_numpy(b.astype(np.float32)),
         "w_down": torch.from_numpy(wd.astype(np.float32)).to(torch.bfloat16)}
    return t


@pytest.mark.parametrize("n,b0", [(2000, -10), (2000, -11), (300, -10), (150, -11), (40, -10)])
def test_forward_integer_valued_exact(n, b0):
    """Every stage on integer-valued data, y bit-exact against the oracle:
    about 20% of the rows dense at b0 = -10, about 2% at b0 = -11 (few live
    fallback tiles, so the fallback splits K over many workgroups), 40 rows
    on the split-K small-batch kernels."""
    dm, dff, T, C = 512, 2048, 128, 4
    say(f"forward integer-valued n={n} b0={b0}")
    t = integer_layer(n + 17 * dff, n, dm, dff, b0)
    d = inputs_to_device(t)
    out = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], T, C,
                                   debug_h=True)
    torch.cuda.synchronize()
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    assert np.max(h_ref) < 16 and np.max(np.abs(y_ref)) < 64
    np.testing.assert_array_equal(as_f64(out.h_debug), h_ref)
    ref = assert_pack_matches(out.hybrid, as_f32(out.h_debug))
    assert 0 < ref.n_dense < n
    np.testing.assert_array_equal(as_f64(out.y), y_ref)
    say(f"  n_dense={ref.n_dense}")


@pytest.mark.parametrize("n_rows,d_model,d_ff", [(64, 128, 512), (45, 72, 320), (33, 512, 2560),
                                                 (7, 264, 1088)])
def test_forward_fp32_small_batch_matches_timed_and_standalone(n_rows, d_model, d_ff):
    """float32, at most 64 rows: the plain call runs the sparse product inside
    the dense-row build (its sparse rows' 16-wave workgroups, one tile range
    per wave), the event-timed variant as its own 16-range kernel. y is the
    same bits both ways; twell_spmm on the standalone pack of the same h gives
    the same bits on the sparse rows (one and several column chunks and tiles
    per range) and runs the dense rows through its own fallback launch
    (checked against the oracle)."""
    cfg = CONFIGS["tiny_fp32"].replace(n_rows=n_rows, d_model=d_model, d_ff=d_ff)
    say(f"fp32 small batch n={n_rows} dm={d_model} dff={d_ff}")
    t = make_inputs(cfg)
    d = inputs_to_device(t)
    a = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                 cfg.capacity, debug_h=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    b = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                 cfg.capacity, stage_events=evs)
    torch.cuda.synchronize()
    assert int(a.status.item()) == twell.TWELL_OK
    assert a.hybrid.n_dense_host() < cfg.n_rows  # some rows go through the sparse product
    hy, _ = twell.twell_pack(a.h_debug, cfg.tile, cfg.capacity)
    y2 = twell.twell_spmm(hy, d["w_down"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(as_f32(a.y)), u32(as_f32(b.y)))
    nd = a.hybrid.n_dense_host()
    sparse = np.ones(cfg.n_rows, dtype=bool)
    sparse[a.hybrid.dense_rows[:nd].cpu().numpy()] = False
    np.testing.assert_array_equal(u32(as_f32(a.y))[sparse], u32(as_f32(y2))[sparse])
    _, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    assert_close_rel(as_f64(a.y), y_ref, TOL[cfg.torch_dtype], "y")
    assert_close_rel(as_f64(y2), y_ref, TOL[cfg.torch_dtype], "twell_spmm y")


@pytest.mark.parametrize("n_rows,d_model,d_ff", [(16, 512, 2048), (48, 512, 2048),
                                                 (700, 512, 2048), (1500, 512, 2048),
                                                 (2600, 512, 2048), (1100, 2048, 8192),
                                                 (3000, 1024, 4096)])
def test_forward_timed_variant_matches_plain_call(n_rows, d_model, d_ff):
    """The event-recording variant (every stage in its own launches) and the
    plain call (at most 64 rows: the sparse product inside the fallback's
    split-K launch) give the same y and hybrid, bit for bit; past 1024 rows
    with one, two and four XCD column slices of the sparse product."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=n_rows, d_model=d_model, d_ff=d_ff)
    say(f"timed vs plain n={n_rows} dm={d_model} dff={d_ff}")
    t = make_inputs(cfg)
    d = inputs_to_device(t)
    a = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                 cfg.capacity)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    b = twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                 cfg.capacity, stage_events=evs)
    torch.cuda.synchronize()
    assert 0 < a.hybrid.n_dense_host() < cfg.n_rows
    np.testing.assert_array_equal(u32(as_f32(a.y)), u32(as_f32(b.y)))
    np.testing.assert_array_equal(a.hybrid.counts.cpu().numpy(), b.hybrid.counts.cpu().numpy())
    np.testing.assert_array_equal(a.hybrid.indices.cpu().numpy(), b.hybrid.indices.cpu().numpy())
    np.testing.assert_array_equal(u32(as_f32(a.hybrid.values)), u32(as_f32(b.hybrid.values)))
    nd = a.hybrid.n_dense_host()
    assert nd == b.hybrid.n_dense_host()
    np.testing.assert_array_equal(a.hybrid.dense_rows[:nd].cpu().numpy(),
                                  b.hybrid.dense_rows[:nd].cpu().numpy())
    np.testing.assert_array_equal(u32(as_f32(a.hybrid.dense_values[:nd])),
                                  u32(as_f32(b.hybrid.dense_values[:nd])))
    assert all(evs[i].elapsed_time(evs[i + 1]) >= 0 for i in range(4))
    _, y_ref = oracle.ffn_forward(*oracle_inputs(t))
    assert_close_rel(as_f64(a.y), y_ref, TOL[cfg.torch_dtype], "y")
