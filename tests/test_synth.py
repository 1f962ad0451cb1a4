"""Determinism and statistical sanity of the seeded input generator."""
import math

import numpy as np
import pytest
import torch
from numpy.random import PCG64, Generator, SeedSequence

from activation_sparse_transformer_amd.synth import CHUNK_ROWS, CONFIGS, draw_normal, make_inputs
from oracle import ffn_hidden, tile_counts


def test_block_layout_is_fixed():
    a = draw_normal(SeedSequence(5), (CHUNK_ROWS + 44, 9))
    kids = SeedSequence(5).spawn(2)
    b0 = Generator(PCG64(kids[0])).standard_normal((CHUNK_ROWS, 9), dtype=np.float32)
    b1 = Generator(PCG64(kids[1])).standard_normal((44, 9), dtype=np.float32)
    np.testing.assert_array_equal(a, np.concatenate([b0, b1]))


def test_deterministic_and_typed():
    cfg = CONFIGS["tiny_fp32"]
    a, b = make_inputs(cfg), make_inputs(cfg)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["x"].dtype == torch.float32 and a["x"].shape == (64, 128)
    assert a["w_up_t"].shape == (512, 128) and a["w_down"].shape == (512, 128)
    assert a["b_up"].dtype == torch.float32 and torch.all(a["b_up"] == np.float32(-1.645))
    small = CONFIGS["ffn_1b_bf16"].replace(n_rows=32, d_model=64, d_ff=256)
    c = make_inputs(small)
    assert c["x"].dtype == torch.bfloat16 and c["w_down"].dtype == torch.bfloat16


def test_bias_noise_and_token_scale():
    cfg = CONFIGS["hybrid_stress_bf16"].replace(n_rows=512, d_model=64, d_ff=4096)
    t = make_inputs(cfg)
    b = t["b_up"].double().numpy()
    assert abs(b.mean() + 2.326) < 0.05 and abs(b.var() - 0.2) < 0.03
    norms = torch.linalg.vector_norm(t["x"].float(), dim=1).double().numpy() / math.sqrt(64)
    # log of the per-token scale has variance 0.5 (plus a little chi noise)
    assert 0.4 < np.log(norms).var() < 0.65


def _phi(z):
    return 0.5 * math.erfc(-z / math.sqrt(2))


@pytest.mark.parametrize("name,rows", [("tiny_fp32", 64), ("ffn_1b_bf16", 128)])
def test_active_fraction(name, rows):
    cfg = CONFIGS[name]
    t = make_inputs(cfg.replace(n_rows=rows))
    h = ffn_hidden(t["x"].double().numpy(), t["w_up_t"].double().numpy(), t["b_up"].double().numpy())
    frac = (h > 0).mean()
    expect = _phi(cfg.b0)
    sigma = math.sqrt(expect * (1 - expect) / h.size)
    assert abs(frac - expect) < 6 * sigma + 0.1 * expect, (frac, expect)


def test_row_overflow_rate_1b():
    # With ~1% active, a T=128 tile holds Binomial(128, 0.01) non-zeros; it
    # overflows C=4 with probability ~0.96%, so a row of 64 tiles goes dense
    # with probability ~46%.  A 128-token sample must land near it.
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=128)
    t = make_inputs(cfg)
    h = ffn_hidden(t["x"].double().numpy(), t["w_up_t"].double().numpy(), t["b_up"].double().numpy())
    dense = (tile_counts(h, cfg.tile) > cfg.capacity).any(axis=1).mean()
    assert 0.30 < dense < 0.62, dense
