"""GPU parity of the layer's backward pass (ffn_sparse_backward) against the
CPU oracle's ffn_backward_from_h, on the same stored activations.

h is the oracle's forward (ReLU(x W_up + b), float64, cast to the storage
type), packed into hybrid TwELL on the GPU by twell_pack (bit-exact against
the oracle's packer in the pack tests); the oracle takes that same h.
Tolerances: 1e-4 (float32) and 1e-2 (bfloat16) of max|ref| per output; the
integer-valued layers are exact (every sum an integer below 2^24, dz an
integer below 2^8, so bfloat16 holds it).  Cases: dense rows (the fallback for
dx, dense-row entries for the weight sums), ragged row counts, 40 rows (the
split-K small-batch fallback), tile widths 64/128/256, a dense capacity below
the dense-row count, 0 rows, run-to-run determinism, and the 1B and decode
layers at full size (dx on sampled rows, weight and bias gradients on sampled
neurons, each computed by the oracle on its own)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_transformer_amd import synth, twell
from gpu_helpers import TOL, as_f32, as_f64, assert_close_rel, oracle_inputs, say

pytestmark = pytest.mark.gpu


def layer(n, dm, dff, T, C, dtype, b0, tsv=0.0, seed=0):
    cfg = synth.FfnConfig("bwd", n, dm, dff, T, C, dtype, b0, token_scale_var=tsv, seed=seed)
    t = synth.make_inputs(cfg)
    t["dy"] = synth.make_grad(cfg)
    return cfg, t


def oracle_h(t, dtype):
    """The oracle's h in the storage type (torch's CPU cast rounds to nearest even)."""
    x, wu, b, _ = oracle_inputs(t)
    return torch.from_numpy(oracle.ffn_hidden(x, wu, b)).to(dtype)


def stored_h(h: np.ndarray, hy: twell.Hybrid) -> np.ndarray:
    """h as the hybrid holds it: rows that went dense past dense_capacity are
    not stored (their slots are cleared), so they read as zero."""
    ref = oracle.pack(h.astype(np.float32), hy.tile, hy.capacity)
    out = h.copy()
    out[ref.dense_rows[hy.dense_capacity:]] = 0.0
    return out


def run_backward(t, h, T, C, dense_capacity=None):
    d = {k: v.cuda() for k, v in t.items()}
    hy, status = twell.twell_pack(h.cuda(), T, C, dense_capacity=dense_capacity)
    g = twell.ffn_sparse_backward(d["x"], d["w_up_t"], d["w_down"], hy, d["dy"])
    torch.cuda.synchronize()
    return hy, int(status.item()), g


def check(g: twell.Grads, ref: oracle.Grads, tol):
    assert_close_rel(as_f64(g.dw_down), ref.dw_down, tol, "dw_down")
    assert_close_rel(as_f64(g.dw_up_t), ref.dw_up_t, tol, "dw_up_t")
    assert_close_rel(as_f64(g.db_up), ref.db, tol, "db_up")
    assert_close_rel(as_f64(g.dx), ref.dx, tol, "dx")


@pytest.mark.parametrize("n,dm,dff,T,C,dtype,b0,tsv", [
    (300, 256, 1024, 64, 4, "bf16", -2.326, 0.5),
    (300, 256, 1024, 64, 4, "fp32", -2.326, 0.5),
    (40, 136, 768, 128, 4, "bf16", -1.645, 0.5),
    (40, 136, 768, 128, 4, "fp32", -1.645, 0.5),
    (500, 512, 2048, 256, 8, "bf16", -1.645, 0.5),
    (1000, 384, 1536, 128, 6, "fp32", -1.645, 0.5),
    (129, 1024, 512, 128, 16, "bf16", -2.326, 0.0),
    # d_model past one pass of the per-neuron kernel: column chunks, ragged
    (100, 2304, 512, 64, 4, "fp32", -1.645, 0.5),
    (70, 4352, 512, 128, 8, "bf16", -1.645, 0.5),
    (90, 4096, 1024, 128, 4, "bf16", -2.326, 0.5),
])
def test_backward_matches_oracle(n, dm, dff, T, C, dtype, b0, tsv):
    say(f"backward {dtype} n={n} dm={dm} dff={dff} T={T} C={C}")
    cfg, t = layer(n, dm, dff, T, C, dtype, b0, tsv, seed=n + dff)
    h = oracle_h(t, cfg.torch_dtype)
    hy, status, g = run_backward(t, h, T, C)
    assert status == twell.TWELL_OK
    x, wu, _, wd = oracle_inputs(t)
    ref = oracle.ffn_backward_from_h(x, as_f64(h), wu, wd, as_f64(t["dy"]))
    if tsv > 0:
        assert 0 < hy.n_dense_host() < n  # both the gather and the fallback run
    check(g, ref, TOL[cfg.torch_dtype])


@pytest.mark.parametrize("cap", [0, 3])
def test_backward_dense_capacity_short(cap):
    """After a dense-capacity overflow the rows past the capacity hold no
    non-zero: no weight-gradient contribution, dx = 0."""
    say(f"backward dense capacity {cap}")
    n, dm, dff, T, C = 300, 256, 1024, 64, 4
    cfg, t = layer(n, dm, dff, T, C, "bf16", -2.326, 0.5, seed=11)
    h = oracle_h(t, torch.bfloat16)
    hy, status, g = run_backward(t, h, T, C, dense_capacity=cap)
    assert status == twell.TWELL_ERR_DENSE_CAPACITY and hy.n_dense_host() > cap
    x, wu, _, wd = oracle_inputs(t)
    hs = stored_h(as_f64(h), hy)
    ref = oracle.ffn_backward_from_h(x, hs, wu, wd, as_f64(t["dy"]))
    check(g, ref, TOL[torch.bfloat16])
    lost = oracle.pack(as_f32(h), T, C).dense_rows[cap:]
    assert len(lost) and not as_f32(g.dx)[lost].any()


def integer_case(seed, n, dm, dff, b0, dtype):
    """x, W_up, W_down, dy in {-1, 0, 1}, an integer bias: h, dz and every
    sum are small integers, exact in float32 accumulation in any order."""
    rng = np.random.default_rng(seed)
    def tern(shape, zero):
        a = rng.integers(-1, 2, size=shape).astype(np.float32)
        a[rng.random(shape) < zero] = 0
        return torch.from_numpy(a).to(dtype)
    return {"x": tern((n, dm), 0.7), "w_up_t": tern((dff, dm), 0.7),
            "b_up": torch.full((dff,), float(b0), dtype=torch.float32),
            "w_down": tern((dff, dm), 0.8), "dy": tern((n, dm), 0.5)}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,b0", [(700, -10), (40, -10), (257, -11)])
def test_backward_integer_valued_exact(dtype, n, b0):
    dm, dff, T, C = 512, 2048, 128, 4
    say(f"backward integer-valued {dtype} n={n} b0={b0}")
    t = integer_case(n + b0 + 7, n, dm, dff, b0, dtype)
    h = oracle_h(t, dtype)
    hy, status, g = run_backward(t, h, T, C)
    assert status == twell.TWELL_OK
    x, wu, _, wd = oracle_inputs(t)
    ref = oracle.ffn_backward_from_h(x, as_f64(h), wu, wd, as_f64(t["dy"]))
    dz = np.where(as_f64(h) != 0, as_f64(t["dy"]) @ wd.T, 0.0)
    assert np.abs(dz).max() <= 256  # dz exact in bfloat16 too
    assert hy.n_dense_host() > 0
    np.testing.assert_array_equal(as_f64(g.dw_down), ref.dw_down)
    np.testing.assert_array_equal(as_f64(g.dw_up_t), ref.dw_up_t)
    np.testing.assert_array_equal(as_f64(g.db_up), ref.db)
    # dx: one rounding of the exact sum to the storage type
    want = torch.from_numpy(ref.dx).to(dtype)
    assert torch.equal(g.dx.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       want.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_backward_zero_rows():
    say("backward n=0")
    dm, dff, T, C = 256, 1024, 128, 4
    d = {k: v.cuda() for k, v in layer(0, dm, dff, T, C, "bf16", -2.0)[1].items()}
    hy, _ = twell.twell_pack(torch.empty((0, dff), dtype=torch.bfloat16, device="cuda"), T, C)
    out = twell.Grads(torch.empty((0, dm), dtype=torch.bfloat16, device="cuda"),
                      torch.full((dff, dm), float("nan"), device="cuda"),
                      torch.full((dff,), float("nan"), device="cuda"),
                      torch.full((dff, dm), float("nan"), device="cuda"))
    g = twell.ffn_sparse_backward(d["x"], d["w_up_t"], d["w_down"], hy, d["dy"], out=out)
    torch.cuda.synchronize()
    for a in (g.dw_up_t, g.db_up, g.dw_down):
        assert torch.equal(a, torch.zeros_like(a))


def test_backward_all_zero_h():
    """No active unit: every gradient is zero (dx too)."""
    say("backward h = 0")
    n, dm, dff, T, C = 100, 256, 1024, 128, 4
    d = {k: v.cuda() for k, v in layer(n, dm, dff, T, C, "bf16", -2.0)[1].items()}
    hy, _ = twell.twell_pack(torch.zeros((n, dff), dtype=torch.bfloat16, device="cuda"), T, C)
    g = twell.ffn_sparse_backward(d["x"], d["w_up_t"], d["w_down"], hy, d["dy"])
    torch.cuda.synchronize()
    for a in (g.dx, g.dw_up_t, g.db_up, g.dw_down):
        assert not a.float().any()


def test_backward_deterministic():
    """Every sum runs in row order: two calls agree bit for bit."""
    say("backward determinism")
    n, dm, dff, T, C = 2000, 512, 2048, 128, 4
    cfg, t = layer(n, dm, dff, T, C, "bf16", -1.645, 0.5, seed=5)
    d = {k: v.cuda() for k, v in t.items()}
    hy, _ = twell.twell_pack(oracle_h(t, torch.bfloat16).cuda(), T, C)
    a = twell.ffn_sparse_backward(d["x"], d["w_up_t"], d["w_down"], hy, d["dy"])
    b = twell.ffn_sparse_backward(d["x"], d["w_up_t"], d["w_down"], hy, d["dy"])
    torch.cuda.synchronize()
    assert hy.n_dense_host() > 0
    for u, v in ((a.dx, b.dx), (a.dw_up_t, b.dw_up_t), (a.db_up, b.db_up),
                 (a.dw_down, b.dw_down)):
        assert torch.equal(u, v)


@pytest.mark.parametrize("name", ["ffn_1b_bf16", "decode_bf16"])
def test_backward_full_size_sampled(name):
    cfg = synth.CONFIGS[name]
    say(f"backward full size {name}")
    t = synth.make_inputs(cfg)
    t["dy"] = synth.make_grad(cfg)
    h = oracle_h(t, cfg.torch_dtype)
    hy, status, g = run_backward(t, h, cfg.tile, cfg.capacity)
    assert status == twell.TWELL_OK
    x, wu, _, wd = oracle_inputs(t)
    hh, dy = as_f64(h), as_f64(t["dy"])
    rng = np.random.default_rng(1)
    tol = TOL[cfg.torch_dtype]
    nd = hy.n_dense_host()
    rows = np.unique(np.concatenate([rng.integers(0, cfg.n_rows, 12), [0, cfg.n_rows - 1],
                                     hy.dense_rows[:min(nd, 4)].cpu().numpy()]))
    ref_rows = oracle.ffn_backward_from_h(x[rows], hh[rows], wu, wd, dy[rows])
    assert_close_rel(as_f64(g.dx)[rows], ref_rows.dx, tol, "dx rows")
    active = (hh != 0).sum(axis=0)
    js = np.unique(np.concatenate([rng.integers(0, cfg.d_ff, 12), [0, cfg.d_ff - 1],
                                   [int(active.argmax())]]))
    ref_cols = oracle.ffn_backward_from_h(x, hh[:, js], wu[js], wd[js], dy)
    assert_close_rel(as_f64(g.dw_down)[js], ref_cols.dw_down, tol, "dw_down neurons")
    assert_close_rel(as_f64(g.dw_up_t)[js], ref_cols.dw_up_t, tol, "dw_up_t neurons")
    assert_close_rel(as_f64(g.db_up)[js], ref_cols.db, tol, "db neurons")
