"""Pins for the oracle's TwELL packer, unpacker and hybrid product.

The pages print no worked example of the format, so every expected value here
comes from the format's definition (values = non-zeros only, tile-local
indices, per-tile counts, tile size T and tile index t, rows split between
TwELL and a dense matrix; "Sparser, Faster, Lighter Transformer Language
Models (Sakana AI + NVIDIA)", Figure 1 description), from invariants that
follow from it, from special cases that reduce to textbook ELLPACK or to a
value-plus-bitmap encoding, or from brute force on tiny inputs.
"""
import numpy as np
import pytest

from oracle import (
    Hybrid, ell_pack_textbook, pack, pack_reference, spmm, tile_counts, to_csr, unpack)


def bits(a):
    a = np.asarray(a)
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def assert_hybrid_identical(a: Hybrid, b: Hybrid):
    assert (a.tile, a.capacity, a.d_ff) == (b.tile, b.capacity, b.d_ff)
    np.testing.assert_array_equal(bits(a.values), bits(b.values))
    np.testing.assert_array_equal(a.indices, b.indices)
    np.testing.assert_array_equal(a.counts, b.counts)
    np.testing.assert_array_equal(a.dense_rows, b.dense_rows)
    assert a.dense_values.shape == b.dense_values.shape
    np.testing.assert_array_equal(bits(a.dense_values), bits(b.dense_values))
    assert a.values.dtype == b.values.dtype and a.dense_values.dtype == b.dense_values.dtype


def check_invariants(h: np.ndarray, hyb: Hybrid):
    """The format's invariants, checked against h itself."""
    n, d_ff = h.shape
    T, C = hyb.tile, hyb.capacity
    nt = d_ff // T
    cnt = tile_counts(h, T)
    dense = (cnt > C).any(axis=1)
    # rows are dense exactly when some tile overflows; listed ascending
    np.testing.assert_array_equal(hyb.dense_rows, np.nonzero(dense)[0])
    assert np.all(np.diff(hyb.dense_rows) > 0)
    for r in range(n):
        if dense[r]:
            assert np.all(hyb.counts[r] == 0)
            assert np.all(bits(hyb.values[r]) == 0) and np.all(hyb.indices[r] == 0)
            continue
        # sum of tile counts = non-zeros of the row; every count <= C
        assert int(hyb.counts[r].sum()) == int((h[r] != 0).sum())
        assert np.all(hyb.counts[r] <= C)
        for t in range(nt):
            c = int(hyb.counts[r, t])
            idx = hyb.indices[r, t, :c].astype(np.int64)
            # indices strictly increasing and < T; they point at the stored values
            assert np.all(np.diff(idx) > 0) and np.all(idx < T)
            np.testing.assert_array_equal(bits(hyb.values[r, t, :c]), bits(h[r, t * T + idx]))
            # padding slots: value +0.0 bits, index 0
            assert np.all(bits(hyb.values[r, t, c:]) == 0) and np.all(hyb.indices[r, t, c:] == 0)
    np.testing.assert_array_equal(bits(hyb.dense_values), bits(h[dense]))


def random_sparse(rng, n, d_ff, density, dtype=np.float32, negzero=False):
    h = rng.standard_normal((n, d_ff)).astype(dtype)
    h[rng.random((n, d_ff)) >= density] = 0
    if negzero:
        z = (h == 0) & (rng.random((n, d_ff)) < 0.5)
        h[z] = -0.0
    return h


# ---------------------------------------------------------------- worked example
def worked_example():
    # 3 token rows, d_ff = 8, T = 4 (two tiles), C = 2.
    h = np.array([
        [0.0, 1.5, 0.0, -2.0, 0.0, 0.0, 0.0, 0.0],   # tiles: 2 nnz, 0 nnz -> sparse
        [3.0, 0.0, 0.0, 0.0, 4.0, 5.0, 6.0, 0.0],    # tile 1 holds 3 > C -> dense
        [-0.0, 0.0, 0.0, 7.0, 0.0, 0.0, 8.0, 0.0],   # -0.0 is zero -> 1 nnz, 1 nnz
    ], dtype=np.float32)
    return h


def test_worked_example_by_hand():
    h = worked_example()
    exp_values = np.array([[[1.5, -2.0], [0, 0]],
                           [[0, 0], [0, 0]],
                           [[7.0, 0], [8.0, 0]]], dtype=np.float32)
    exp_indices = np.array([[[1, 3], [0, 0]],
                            [[0, 0], [0, 0]],
                            [[3, 0], [2, 0]]], dtype=np.uint8)
    exp_counts = np.array([[2, 0], [0, 0], [1, 1]], dtype=np.uint8)
    for packer in (pack_reference, pack):
        hyb = packer(h, 4, 2)
        np.testing.assert_array_equal(bits(hyb.values), bits(exp_values))
        np.testing.assert_array_equal(hyb.indices, exp_indices)
        np.testing.assert_array_equal(hyb.counts, exp_counts)
        np.testing.assert_array_equal(hyb.dense_rows, [1])
        np.testing.assert_array_equal(hyb.dense_values, h[1:2])
        # unpack: the -0.0 of row 2 comes back as +0.0, everything else bitwise
        u = unpack(hyb)
        exp_u = h.copy()
        exp_u[2, 0] = 0.0
        np.testing.assert_array_equal(bits(u), bits(exp_u))


def test_worked_example_spmm_by_hand():
    h = worked_example()
    hyb = pack(h, 4, 2)
    # W_down [8, 2]: row j = (j, 1)
    w = np.stack([np.arange(8.0), np.ones(8)], axis=1)
    y = spmm(hyb, w)
    # row0: 1.5*(1,1) + -2*(3,1) = (-4.5, -0.5)
    # row1: 3*(0,1) + 4*(4,1) + 5*(5,1) + 6*(6,1) = (77, 18)
    # row2: 7*(3,1) + 8*(6,1) = (69, 15)
    np.testing.assert_array_equal(y, [[-4.5, -0.5], [77.0, 18.0], [69.0, 15.0]])


# ------------------------------------------------------------ reference vs fast
@pytest.mark.parametrize("T,C", [(4, 1), (4, 2), (8, 3), (16, 4), (32, 8), (64, 8), (64, 64)])
@pytest.mark.parametrize("density", [0.02, 0.1, 0.3])
def test_vectorized_matches_reference(T, C, density):
    rng = np.random.default_rng(1000 * T + C + int(density * 100))
    n, d_ff = 37, T * 5
    h = random_sparse(rng, n, d_ff, density, negzero=True)
    a = pack_reference(h, T, C)
    b = pack(h, T, C, chunk_rows=8)  # several chunks and a ragged last one
    assert_hybrid_identical(a, b)
    check_invariants(h, b)


def test_vectorized_matches_reference_float64_and_bf16_grid():
    rng = np.random.default_rng(7)
    # values on the bf16 grid, held as float32 (as the tests hold GPU output)
    h = random_sparse(rng, 20, 256, 0.05)
    h = (h.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    assert_hybrid_identical(pack_reference(h, 128, 4), pack(h, 128, 4))
    h64 = random_sparse(rng, 11, 192, 0.1, dtype=np.float64)
    assert_hybrid_identical(pack_reference(h64, 64, 5), pack(h64, 64, 5))


# ------------------------------------------------------------------- invariants
@pytest.mark.parametrize("T,C,density", [(64, 8, 0.05), (128, 4, 0.01), (128, 4, 0.03), (256, 8, 0.1)])
def test_invariants_random(T, C, density):
    rng = np.random.default_rng(T + C)
    h = random_sparse(rng, 300, T * 6, density)
    hyb = pack(h, T, C)
    check_invariants(h, hyb)
    # round trip is bitwise when zeros are +0.0
    np.testing.assert_array_equal(bits(unpack(hyb)), bits(h))


def test_round_trip_negative_zero_by_value():
    rng = np.random.default_rng(3)
    h = random_sparse(rng, 50, 128, 0.05, negzero=True)
    hyb = pack(h, 64, 3)
    u = unpack(hyb)
    np.testing.assert_array_equal(u, h)  # by value
    dense = np.zeros(50, bool)
    dense[hyb.dense_rows] = True
    # sparse rows: every zero comes back as +0.0; dense rows: copied bitwise
    assert np.all(bits(u[~dense][u[~dense] == 0]) == 0)
    np.testing.assert_array_equal(bits(u[dense]), bits(h[dense]))


# ---------------------------------------------------------------- special cases
def test_capacity_equal_tile_never_dense():
    rng = np.random.default_rng(5)
    h = random_sparse(rng, 40, 4 * 32, 0.9)
    hyb = pack(h, 32, 32)
    assert hyb.n_dense == 0
    np.testing.assert_array_equal(hyb.counts, tile_counts(h, 32))
    np.testing.assert_array_equal(bits(unpack(hyb)), bits(h))


def test_single_tile_is_textbook_ellpack():
    # T = d_ff: one tile per row, so TwELL is ELLPACK of width C (Figure 1(a)).
    rng = np.random.default_rng(11)
    d_ff, C = 96, 6
    h = random_sparse(rng, 60, d_ff, 0.04)
    nnz = (h != 0).sum(1)
    hyb = pack(h, d_ff, C)
    fit = nnz <= C
    assert fit.any() and (~fit).any()
    vals, cols, ell_nnz = ell_pack_textbook(h[fit], C)
    np.testing.assert_array_equal(bits(hyb.values[fit, 0, :]), bits(vals))
    np.testing.assert_array_equal(hyb.indices[fit, 0, :], cols)
    np.testing.assert_array_equal(hyb.counts[fit, 0], ell_nnz)
    np.testing.assert_array_equal(hyb.dense_rows, np.nonzero(~fit)[0])
    with pytest.raises(ValueError):
        ell_pack_textbook(h[~fit], C)


def test_tile_one_capacity_one_is_value_plus_bitmap():
    rng = np.random.default_rng(13)
    h = random_sparse(rng, 25, 40, 0.3, negzero=True)
    hyb = pack(h, 1, 1)
    assert hyb.n_dense == 0
    np.testing.assert_array_equal(hyb.counts[:, :], (h != 0).astype(np.uint8))
    assert np.all(hyb.indices == 0)
    expect = np.where(h != 0, h, np.float32(0.0))  # -0.0 becomes +0.0 padding
    np.testing.assert_array_equal(bits(hyb.values[:, :, 0]), bits(expect))


def test_all_zero_and_all_positive():
    z = np.zeros((5, 256), np.float32)
    hz = pack(z, 128, 4)
    assert hz.n_dense == 0 and np.all(hz.counts == 0) and np.all(bits(hz.values) == 0)
    p = np.full((5, 256), 2.5, np.float32)
    hp = pack(p, 128, 4)
    np.testing.assert_array_equal(hp.dense_rows, np.arange(5))
    np.testing.assert_array_equal(hp.dense_values, p)
    assert np.all(hp.counts == 0)


def test_exactly_capacity_and_one_more():
    T, C = 64, 8
    h = np.zeros((3, 3 * T), np.float32)
    h[0, T + np.arange(C) * 7] = 1.0          # exactly C in tile 1 -> sparse
    h[1, 2 * T + np.arange(C + 1) * 7] = 1.0  # C+1 in the last tile -> dense
    h[2, 3 * T - 1] = 9.0                     # last column only
    hyb = pack(h, T, C)
    np.testing.assert_array_equal(hyb.dense_rows, [1])
    np.testing.assert_array_equal(hyb.counts[0], [0, C, 0])
    np.testing.assert_array_equal(hyb.indices[0, 1], np.arange(C) * 7)
    np.testing.assert_array_equal(hyb.counts[2], [0, 0, 1])
    assert hyb.indices[2, 2, 0] == T - 1 and hyb.values[2, 2, 0] == 9.0


def test_nan_counts_as_nonzero():
    h = np.zeros((2, 8), np.float32)
    h[0, 2] = np.nan
    h[1, [0, 1, 2]] = np.nan
    hyb = pack(h, 4, 2)
    assert hyb.counts[0, 0] == 1 and hyb.indices[0, 0, 0] == 2 and np.isnan(hyb.values[0, 0, 0])
    np.testing.assert_array_equal(hyb.dense_rows, [1])
    assert_hybrid_identical(hyb, pack_reference(h, 4, 2))


def test_zero_rows():
    h = np.zeros((0, 256), np.float32)
    for packer in (pack, pack_reference):
        hyb = packer(h, 128, 4)
        assert hyb.values.shape == (0, 2, 4) and hyb.n_dense == 0
        assert unpack(hyb).shape == (0, 256)
        assert spmm(hyb, np.ones((256, 3))).shape == (0, 3)


def test_geometry_checks():
    h = np.zeros((2, 100), np.float32)
    with pytest.raises(ValueError):
        pack(h, 64, 4)  # 64 does not divide 100
    with pytest.raises(ValueError):
        pack(np.zeros((2, 128)), 64, 65)  # C > T
    with pytest.raises(ValueError):
        pack(np.zeros((2, 512)), 512, 4)  # T > 256


# ------------------------------------------------------------------------ spmm
def brute_spmm(hyb: Hybrid, w):
    n, nt, C = hyb.values.shape
    dm = w.shape[1]
    y = [[0.0] * dm for _ in range(n)]
    for r in range(n):
        for t in range(nt):
            for k in range(int(hyb.counts[r, t])):
                j = t * hyb.tile + int(hyb.indices[r, t, k])
                for c in range(dm):
                    y[r][c] += float(hyb.values[r, t, k]) * float(w[j, c])
    for m, r in enumerate(hyb.dense_rows):
        for j in range(hyb.d_ff):
            for c in range(dm):
                y[r][c] += float(hyb.dense_values[m, j]) * float(w[j, c])
    return np.array(y)


def test_spmm_integer_exact_vs_brute_force():
    rng = np.random.default_rng(17)
    h = rng.integers(-3, 4, size=(12, 48)).astype(np.float32)
    h[rng.random(h.shape) < 0.8] = 0
    w = rng.integers(-5, 6, size=(48, 7)).astype(np.float64)
    hyb = pack(h, 16, 3)
    assert 0 < hyb.n_dense < 12
    np.testing.assert_array_equal(spmm(hyb, w), brute_spmm(hyb, w))


def test_spmm_identity_is_unpack():
    rng = np.random.default_rng(19)
    h = random_sparse(rng, 30, 128, 0.06)
    hyb = pack(h, 64, 4)
    assert hyb.n_dense > 0
    np.testing.assert_array_equal(spmm(hyb, np.eye(128)), unpack(hyb).astype(np.float64))


def test_spmm_matches_dense_product():
    rng = np.random.default_rng(23)
    h = random_sparse(rng, 64, 512, 0.05)
    w = rng.standard_normal((512, 40))
    hyb = pack(h, 64, 4)
    np.testing.assert_allclose(spmm(hyb, w), h.astype(np.float64) @ w, rtol=1e-12, atol=1e-12)


def test_to_csr_holds_only_sparse_rows():
    h = worked_example()
    m = to_csr(pack(h, 4, 2)).toarray()
    assert np.all(m[1] == 0)
    np.testing.assert_array_equal(m[[0, 2]], np.abs(h[[0, 2]]) * np.sign(h[[0, 2]]))
