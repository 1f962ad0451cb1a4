"""Pins for the oracle's dense FFN and its bfloat16 decoder.

The FFN is the plain non-gated ReLU feed-forward layer y = ReLU(x W_up + b)
W_down ("The Relentless Search for Efficiency in Large-Scale Language Models",
section "The Challenge of Sparsity Ignored by GPUs").  Pins: closed forms
(a permutation up-projection with a diagonal down-projection, a hand-computed
2-token example), brute force on tiny inputs, the two bias limits, positive
homogeneity and row-permutation equivariance.
"""
import math

import numpy as np
import torch

from oracle import bf16_bits_to_f32, ffn_forward, ffn_forward_rows, ffn_hidden


def test_hand_computed_example():
    # d_model = 3, d_ff = 2, d_model_out = 3
    x = np.array([[1.0, 2.0, -1.0],
                  [0.5, -1.0, 4.0]])
    w_up_t = np.array([[1.0, 0.0, 1.0],    # neuron 0: x0 + x2
                       [0.0, 1.0, -1.0]])  # neuron 1: x1 - x2
    b = np.array([0.5, -4.0])
    w_down = np.array([[1.0, 2.0, 3.0],
                       [-1.0, 0.0, 1.0]])
    # token 0: z = (0 + 0.5, 3 - 4) = (0.5, -1) -> h = (0.5, 0) -> y = (0.5, 1, 1.5)
    # token 1: z = (4.5 + 0.5, -5 - 4) = (5, -9) -> h = (5, 0)  -> y = (5, 10, 15)
    h, y = ffn_forward(x, w_up_t, b, w_down)
    np.testing.assert_array_equal(h, [[0.5, 0.0], [5.0, 0.0]])
    np.testing.assert_array_equal(y, [[0.5, 1.0, 1.5], [5.0, 10.0, 15.0]])


def test_permutation_up_diagonal_down_closed_form():
    rng = np.random.default_rng(0)
    n, d = 9, 13
    perm = rng.permutation(d)
    w_up_t = np.zeros((d, d))
    w_up_t[np.arange(d), perm] = 1.0          # z[:, j] = x[:, perm[j]] + b[j]
    diag = rng.standard_normal(d)
    w_down = np.diag(diag)                      # y[:, k] = diag[k] * h[:, k]
    x = rng.standard_normal((n, d))
    b = rng.standard_normal(d)
    h, y = ffn_forward(x, w_up_t, b, w_down)
    expect_h = np.maximum(x[:, perm] + b, 0.0)
    np.testing.assert_array_equal(h, expect_h)
    np.testing.assert_array_equal(y, expect_h * diag)


def test_brute_force_tiny():
    rng = np.random.default_rng(1)
    n, dm, dff = 4, 5, 7
    x = rng.standard_normal((n, dm))
    w_up_t = rng.standard_normal((dff, dm))
    b = rng.standard_normal(dff)
    w_down = rng.standard_normal((dff, dm))
    h, y = ffn_forward(x, w_up_t, b, w_down)
    for r in range(n):
        hid = []
        for j in range(dff):
            z = b[j]
            for i in range(dm):
                z += x[r, i] * w_up_t[j, i]
            hid.append(z if z > 0 else 0.0)
        for k in range(dm):
            acc = 0.0
            for j in range(dff):
                acc += hid[j] * w_down[j, k]
            assert math.isclose(y[r, k], acc, rel_tol=1e-12, abs_tol=1e-12)
        np.testing.assert_allclose(h[r], hid, rtol=1e-12, atol=1e-12)


def test_bias_limits():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 16))
    w_up_t = rng.standard_normal((32, 16)) / 4
    w_down = rng.standard_normal((32, 16))
    h, y = ffn_forward(x, w_up_t, np.full(32, -1e4), w_down)
    assert np.all(h == 0) and np.all(y == 0)
    # a huge positive bias keeps every unit: h = z exactly
    h, y = ffn_forward(x, w_up_t, np.full(32, 1e4), w_down)
    assert np.all(h > 0)
    np.testing.assert_allclose(h - 1e4, x @ w_up_t.T, atol=1e-9)


def test_positive_homogeneity_and_row_permutation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 12))
    w_up_t = rng.standard_normal((20, 12))
    b = rng.standard_normal(20)
    w_down = rng.standard_normal((20, 12))
    _, y = ffn_forward(x, w_up_t, b, w_down)
    _, y2 = ffn_forward(4.0 * x, w_up_t, 4.0 * b, w_down)
    np.testing.assert_allclose(y2, 4.0 * y, rtol=1e-13, atol=1e-13)
    p = rng.permutation(10)
    _, yp = ffn_forward(x[p], w_up_t, b, w_down)
    np.testing.assert_allclose(yp, y[p], rtol=1e-13, atol=1e-13)
    _, yr = ffn_forward_rows(x, w_up_t, b, w_down, [7, 2])
    np.testing.assert_allclose(yr, y[[7, 2]], rtol=1e-13, atol=1e-13)


def test_relu_output_is_positive_zero():
    x = np.array([[1.0, -1.0]])
    h = ffn_hidden(x, np.eye(2), np.zeros(2))
    assert np.signbit(h).sum() == 0


def test_bf16_decoder_known_values():
    cases = {
        0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3E20: 0.15625,
        0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: math.inf,
    }
    for b, v in cases.items():
        assert bf16_bits_to_f32(np.array([b], np.uint16))[0] == np.float32(v)
    z = bf16_bits_to_f32(np.array([0x8000], np.uint16))[0]
    assert z == 0 and np.signbit(z)
    assert np.isnan(bf16_bits_to_f32(np.array([0x7FC0], np.uint16))[0])


def test_bf16_decoder_matches_torch_on_every_pattern():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
