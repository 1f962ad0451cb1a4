"""Pins of the oracle's ELL rows (Figure 1(a) with the hybrid split), against
things other than the function itself: a worked example by hand, the
independent textbook ELLPACK packer where every row fits, the TwELL packer
with one tile spanning the row (the same format by construction), and the
format's invariants."""
import numpy as np
import pytest

import oracle


def test_hand_example():
    # width 2: row 0 fits (columns 1 and 4), row 1 has three non-zeros -> dense,
    # row 2 is empty, row 3 holds -0.0 (zero) and one value
    h = np.array([[0, 3, 0, 0, 5, 0],
                  [1, 0, 2, 0, 0, 4],
                  [0, 0, 0, 0, 0, 0],
                  [-0.0, 0, 0, 7, 0, 0]], dtype=np.float32)
    e = oracle.ell_pack(h, 2)
    np.testing.assert_array_equal(e.counts, [2, 0, 0, 1])
    np.testing.assert_array_equal(e.columns, [[1, 4], [0, 0], [0, 0], [3, 0]])
    np.testing.assert_array_equal(e.values, [[3, 5], [0, 0], [0, 0], [7, 0]])
    np.testing.assert_array_equal(e.dense_rows, [1])
    np.testing.assert_array_equal(e.dense_values, h[[1]])
    back = oracle.ell_unpack(e)
    np.testing.assert_array_equal(back, np.abs(h) * np.sign(h) + 0.0)  # -0.0 comes back +0.0
    assert not np.signbit(back[3, 0])


def random_h(seed, n, d, density):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, d)).astype(np.float32)
    h[rng.random((n, d)) >= density] = 0
    return h


@pytest.mark.parametrize("n,d,density", [(30, 200, 0.05), (17, 64, 0.3), (40, 1000, 0.01)])
def test_matches_textbook_when_every_row_fits(n, d, density):
    h = random_h(n + d, n, d, density)
    width = int((h != 0).sum(axis=1).max())
    e = oracle.ell_pack(h, max(width, 1))
    vals, cols, nnz = oracle.ell_pack_textbook(h, max(width, 1))
    assert e.n_dense == 0
    np.testing.assert_array_equal(e.counts, nnz)
    np.testing.assert_array_equal(e.columns, cols)
    np.testing.assert_array_equal(e.values.view(np.uint32), vals.view(np.uint32))


@pytest.mark.parametrize("d,width", [(64, 3), (128, 5), (256, 8), (96, 1)])
def test_is_twell_with_one_tile(d, width):
    """TwELL with T = d_ff is ELL: same slots, same counts, same dense rows."""
    h = random_h(d + width, 50, d, 0.04)
    e = oracle.ell_pack(h, width)
    t = oracle.pack_reference(h, d, width)
    assert 0 < e.n_dense < 50
    np.testing.assert_array_equal(e.counts, t.counts[:, 0])
    np.testing.assert_array_equal(e.columns, t.indices[:, 0, :].astype(np.int64))
    np.testing.assert_array_equal(e.values.view(np.uint32), t.values[:, 0, :].view(np.uint32))
    np.testing.assert_array_equal(e.dense_rows, t.dense_rows)
    np.testing.assert_array_equal(e.dense_values.view(np.uint32), t.dense_values.view(np.uint32))


@pytest.mark.parametrize("width", [1, 4, 9, 40])
def test_invariants_and_round_trip(width):
    h = random_h(width, 60, 300, 0.02)
    z = np.argwhere(h == 0)[::7]
    h[z[:, 0], z[:, 1]] = -0.0
    h[5, 17] = np.nan
    assert np.signbit(h[z[0, 0], z[0, 1]])
    e = oracle.ell_pack(h, width)
    nnz = (h != 0).sum(axis=1)
    dense = nnz > width
    np.testing.assert_array_equal(e.dense_rows, np.nonzero(dense)[0])
    for r in range(60):
        c = int(e.counts[r])
        if dense[r]:
            assert c == 0 and not e.values[r].any() and not e.columns[r].any()
            continue
        assert c == nnz[r]
        assert np.all(np.diff(e.columns[r, :c]) > 0)          # strictly ascending
        assert np.all(e.columns[r, c:] == 0) and np.all(e.values[r, c:].view(np.uint32) == 0)
    back = oracle.ell_unpack(e)
    same = (back.view(np.uint32) == h.view(np.uint32)) | ((h == 0) & (back == 0))
    assert same.all()


def test_width_out_of_range():
    with pytest.raises(ValueError):
        oracle.ell_pack(np.zeros((2, 8), np.float32), 9)
