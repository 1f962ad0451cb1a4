"""Pins of the oracle's ReLU-gated FFN against things other than its own
formula: a hand-worked example, the plain FFN when the up branch is the
constant 1, a brute-force triple loop, exact scaling of the up branch by a
power of two, and the gate's zero set."""
import numpy as np

import oracle


def test_hand_example():
    # d_model 2, d_ff 3, one token x = (1, 2)
    x = np.array([[1.0, 2.0]])
    w_gate_t = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    b_gate = np.array([0.0, -3.0, 1.0])        # gate z = (1, -1, 4): ReLU -> (1, 0, 4)
    w_up_t = np.array([[2.0, 0.0], [1.0, 1.0], [0.0, -1.0]])
    b_up = np.array([1.0, 0.0, 0.5])           # up = (3, 3, -1.5)
    w_down = np.array([[1.0, 0.0], [5.0, 5.0], [0.0, 2.0]])
    h, y = oracle.gated_ffn_forward(x, w_gate_t, b_gate, w_up_t, b_up, w_down)
    np.testing.assert_array_equal(h, [[3.0, 0.0, -6.0]])
    np.testing.assert_array_equal(y, [[3.0, -12.0]])


def test_constant_up_branch_is_the_plain_ffn():
    rng = np.random.default_rng(1)
    n, dm, dff = 5, 8, 12
    x = rng.standard_normal((n, dm))
    w_gate_t = rng.standard_normal((dff, dm))
    b_gate = rng.standard_normal(dff)
    w_down = rng.standard_normal((dff, dm))
    h, y = oracle.gated_ffn_forward(x, w_gate_t, b_gate, np.zeros((dff, dm)), np.ones(dff), w_down)
    h0, y0 = oracle.ffn_forward(x, w_gate_t, b_gate, w_down)
    np.testing.assert_array_equal(h, h0)
    np.testing.assert_array_equal(y, y0)


def test_brute_force_loops():
    rng = np.random.default_rng(2)
    n, dm, dff = 3, 4, 5
    x = rng.integers(-2, 3, (n, dm)).astype(float)
    wg = rng.integers(-2, 3, (dff, dm)).astype(float)
    bg = rng.integers(-2, 3, dff).astype(float)
    wu = rng.integers(-2, 3, (dff, dm)).astype(float)
    bu = rng.integers(-2, 3, dff).astype(float)
    wd = rng.integers(-2, 3, (dff, dm)).astype(float)
    want_y = np.zeros((n, dm))
    for r in range(n):
        for j in range(dff):
            g = sum(x[r, i] * wg[j, i] for i in range(dm)) + bg[j]
            u = sum(x[r, i] * wu[j, i] for i in range(dm)) + bu[j]
            hj = (g if g > 0 else 0.0) * u
            for k in range(dm):
                want_y[r, k] += hj * wd[j, k]
    _, y = oracle.gated_ffn_forward(x, wg, bg, wu, bu, wd)
    np.testing.assert_array_equal(y, want_y)


def test_up_branch_scales_exactly():
    rng = np.random.default_rng(3)
    n, dm, dff = 4, 6, 10
    args = [rng.standard_normal(s) for s in ((n, dm), (dff, dm), (dff,), (dff, dm), (dff,), (dff, dm))]
    x, wg, bg, wu, bu, wd = args
    _, y1 = oracle.gated_ffn_forward(x, wg, bg, wu, bu, wd)
    _, y4 = oracle.gated_ffn_forward(x, wg, bg, 4.0 * wu, 4.0 * bu, wd)
    np.testing.assert_array_equal(y4, 4.0 * y1)


def test_gate_zero_set():
    rng = np.random.default_rng(4)
    n, dm, dff = 20, 16, 64
    x = rng.standard_normal((n, dm))
    wg = rng.standard_normal((dff, dm))
    bg = rng.standard_normal(dff) - 1.0
    wu = rng.standard_normal((dff, dm))
    bu = rng.standard_normal(dff)
    h = oracle.gated_ffn_hidden(x, wg, bg, wu, bu)
    zg = x @ wg.T + bg
    assert np.all(h[zg <= 0] == 0)
    assert np.all(h[zg > 0] != 0)  # the up branch is non-zero almost surely
    # a fully closed gate gives a zero layer
    _, y = oracle.gated_ffn_forward(x, wg, np.full(dff, -1e4), wu, bu, rng.standard_normal((dff, dm)))
    assert not y.any()
