"""Pins of the oracle's backward pass and of its sampled product, against
things other than the formulas themselves: a hand-worked example, central
finite differences of the scalar L = sum(y * dy) away from ReLU kinks,
torch's automatic differentiation on the CPU in float64, the two bias
limits, and the dense product a b^T read at the stored positions."""
import numpy as np
import pytest
import torch

import oracle


def test_hand_example():
    # d_model 2, d_ff 2: token z = (x0 + 1, x1 - 5) -> only neuron 0 active
    x = np.array([[1.0, 2.0]])
    w_up_t = np.array([[1.0, 0.0], [0.0, 1.0]])
    b = np.array([1.0, -5.0])
    w_down = np.array([[2.0, 3.0], [4.0, 5.0]])
    dy = np.array([[1.0, -1.0]])
    g = oracle.ffn_backward(x, w_up_t, b, w_down, dy)
    # h = (2, 0); y = 2 * (2, 3); dW_down = h^T dy = [[2, -2], [0, 0]]
    np.testing.assert_array_equal(g.dw_down, [[2.0, -2.0], [0.0, 0.0]])
    # dh = dy W_down^T = (2 - 3, 4 - 5) = (-1, -1); dz = (-1, 0)
    np.testing.assert_array_equal(g.db, [-1.0, 0.0])
    np.testing.assert_array_equal(g.dw_up_t, [[-1.0, -2.0], [0.0, 0.0]])
    np.testing.assert_array_equal(g.dx, [[-1.0, 0.0]])


def loss(x, w_up_t, b, w_down, dy):
    _, y = oracle.ffn_forward(x, w_up_t, b, w_down)
    return float(np.sum(y * dy))


def test_central_differences():
    rng = np.random.default_rng(4)
    n, dm, dff = 3, 4, 6
    x = rng.standard_normal((n, dm))
    w_up_t = rng.standard_normal((dff, dm))
    b = rng.standard_normal(dff)
    w_down = rng.standard_normal((dff, dm))
    dy = rng.standard_normal((n, dm))
    z = x @ w_up_t.T + b
    assert np.min(np.abs(z)) > 1e-3  # no ReLU kink within the step
    g = oracle.ffn_backward(x, w_up_t, b, w_down, dy)
    eps = 1e-6
    for name, arr, grad in (("x", x, g.dx), ("w_up_t", w_up_t, g.dw_up_t), ("b", b, g.db),
                            ("w_down", w_down, g.dw_down)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(x, w_up_t, b, w_down, dy)
            arr[idx] = old - eps
            lm = loss(x, w_up_t, b, w_down, dy)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_matches_torch_autograd():
    rng = np.random.default_rng(5)
    n, dm, dff = 7, 16, 48
    arrs = [rng.standard_normal(s) for s in ((n, dm), (dff, dm), (dff,), (dff, dm), (n, dm))]
    x, w_up_t, b, w_down, dy = arrs
    g = oracle.ffn_backward(x, w_up_t, b, w_down, dy)
    tx, tw, tb, td = (torch.tensor(a, requires_grad=True) for a in (x, w_up_t, b, w_down))
    y = torch.relu(tx @ tw.T + tb) @ td
    (y * torch.tensor(dy)).sum().backward()
    for ours, ref in ((g.dx, tx.grad), (g.dw_up_t, tw.grad), (g.db, tb.grad), (g.dw_down, td.grad)):
        np.testing.assert_allclose(ours, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_bias_limits():
    rng = np.random.default_rng(6)
    x, w_up_t, w_down, dy = (rng.standard_normal(s) for s in ((5, 8), (12, 8), (12, 8), (5, 8)))
    g = oracle.ffn_backward(x, w_up_t, np.full(12, -1e4), w_down, dy)
    for a in (g.dx, g.dw_up_t, g.db, g.dw_down):
        assert np.all(a == 0)
    # every unit on: the layer is linear, y = (x W_up^T + b) W_down
    b = np.full(12, 1e4)
    g = oracle.ffn_backward(x, w_up_t, b, w_down, dy)
    np.testing.assert_allclose(g.dx, dy @ w_down.T @ w_up_t, rtol=1e-12)
    np.testing.assert_allclose(g.dw_down, (x @ w_up_t.T + b).T @ dy, rtol=1e-12)


@pytest.mark.parametrize("tile,cap", [(8, 2), (16, 3)])
def test_sampled_dots_equal_the_dense_product_at_stored_positions(tile, cap):
    rng = np.random.default_rng(tile + cap)
    n, dff, dm = 20, 64, 9
    h = rng.standard_normal((n, dff))
    h[rng.random((n, dff)) > 0.15] = 0
    a = rng.standard_normal((n, dm))
    bmat = rng.standard_normal((dff, dm))
    hyb = oracle.pack_reference(h, tile, cap)
    assert 0 < hyb.n_dense < n
    vals, dense = oracle.sampled_dots(hyb, a, bmat)
    full = np.where(h != 0, a @ bmat.T, 0.0)
    # the sampled values, put back in place, are the masked dense product
    back = oracle.unpack(oracle.Hybrid(tile, cap, dff, vals, hyb.indices, hyb.counts,
                                       hyb.dense_rows, dense))
    np.testing.assert_allclose(back, full, rtol=1e-12, atol=1e-12)
    # and the backward's dz is that product with a = dy, b = W_down
    g_from_h = oracle.ffn_backward_from_h(rng.standard_normal((n, dm)), h,
                                          rng.standard_normal((dff, dm)), bmat, a)
    np.testing.assert_allclose(g_from_h.db, full.sum(axis=0), rtol=1e-12, atol=1e-12)
