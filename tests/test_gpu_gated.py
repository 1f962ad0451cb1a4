"""GPU parity of the ReLU-gated forward (ffn_sparse_gated_forward) against the
CPU oracle's gated_ffn_forward.

y within 1e-4 (float32) / 1e-2 (bfloat16) of max|y|, and h (the hybrid,
unpacked) within the same bound of max|h|, on layers with dense rows (the
fallback and the up branch at the stored dense rows' non-zeros), ragged row
counts, 40 rows (the split-K small-batch kernels), tile widths 64/128/256
and a d_model that is not a multiple of the vector width of one wave.
Integer-valued layers are exact: the gate's pattern gives counts, indices,
the dense-row list bit for bit against the oracle's packer, and h and y
equal the oracle's values rounded once to the storage type."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_transformer_amd import synth, twell
from gpu_helpers import TOL, as_f32, as_f64, assert_close_rel, say

pytestmark = pytest.mark.gpu
ORDER = ("x", "w_gate_t", "b_gate", "w_up_t", "b_up", "w_down")


def run(t, T, C, dense_capacity=None):
    d = {k: v.cuda() for k, v in t.items()}
    out = twell.ffn_sparse_gated_forward(*(d[k] for k in ORDER), T, C,
                                         dense_capacity=dense_capacity)
    torch.cuda.synchronize()
    return out


def ref(t):
    return oracle.gated_ffn_forward(*(as_f64(t[k]) for k in ORDER))


@pytest.mark.parametrize("n,dm,dff,T,C,dtype,b0,tsv", [
    (300, 256, 1024, 64, 4, "bf16", -2.326, 0.5),
    (300, 256, 1024, 64, 4, "fp32", -2.326, 0.5),
    (40, 136, 768, 128, 4, "bf16", -1.645, 0.5),
    (40, 136, 768, 128, 4, "fp32", -1.645, 0.5),
    (500, 512, 2048, 256, 8, "bf16", -1.645, 0.5),
    (1000, 384, 1536, 128, 6, "fp32", -1.645, 0.5),
    (129, 1024, 512, 128, 16, "bf16", -2.326, 0.0),
    (90, 4096, 1024, 128, 4, "bf16", -2.326, 0.5),
    (600, 512, 4096, 128, 4, "bf16", -2.326, 0.5),   # the up branch mapped by XCD
    (600, 512, 4096, 128, 4, "fp32", -2.326, 0.5),
])
def test_gated_matches_oracle(n, dm, dff, T, C, dtype, b0, tsv):
    say(f"gated forward {dtype} n={n} dm={dm} dff={dff} T={T} C={C}")
    cfg = synth.FfnConfig("gated", n, dm, dff, T, C, dtype, b0, token_scale_var=tsv, seed=n + dm)
    t = synth.make_gated_inputs(cfg)
    out = run(t, T, C)
    assert int(out.status.item()) == twell.TWELL_OK
    h_ref, y_ref = ref(t)
    tol = TOL[cfg.torch_dtype]
    assert_close_rel(as_f64(out.y), y_ref, tol, "y")
    assert_close_rel(as_f64(twell.twell_unpack(out.hybrid)), h_ref, tol, "h")
    if tsv > 0:
        assert 0 < out.hybrid.n_dense_host() < n


def integer_case(seed, n, dm, dff, b0, dtype):
    """x, both weights and W_down in {-1, 0, 1}, integer gate bias, up bias 0:
    the gate, the up branch, h and y are small integers (|h| < 256), exact in
    bfloat16 storage and float32 accumulation in any order."""
    rng = np.random.default_rng(seed)

    def tern(shape, zero):
        a = rng.integers(-1, 2, size=shape).astype(np.float32)
        a[rng.random(shape) < zero] = 0
        return torch.from_numpy(a).to(dtype)
    return {"x": tern((n, dm), 0.7), "w_gate_t": tern((dff, dm), 0.7),
            "b_gate": torch.full((dff,), float(b0)), "w_up_t": tern((dff, dm), 0.8),
            "b_up": torch.zeros(dff), "w_down": tern((dff, dm), 0.8)}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,b0,dff", [(700, -10, 2048), (40, -10, 2048), (257, -11, 2048),
                                      (700, -10, 4096)])
def test_gated_integer_valued_exact(dtype, n, b0, dff):
    """Exact h and y; the up branch's work mapped by XCD (a row's 16 or 32
    tiles in eighths, at least 8 dense chunks: float32 at d_ff 2048, both
    types at 4096) and in 64-slot parts (bfloat16 at 2048)."""
    dm, T, C = 512, 128, 4
    say(f"gated integer-valued {dtype} n={n} b0={b0} dff={dff}")
    t = integer_case(n * 3 + b0, n, dm, dff, b0, dtype)
    out = run(t, T, C)
    h_ref, y_ref = ref(t)
    assert np.abs(h_ref).max() < 256 and np.abs(y_ref).max() < 2 ** 24
    # the stored places are the gate's non-zeros: the oracle's packer on the gate
    x, wg, bg = as_f64(t["x"]), as_f64(t["w_gate_t"]), as_f64(t["b_gate"])
    gate = oracle.ffn_hidden(x, wg, bg)
    pk = oracle.pack(gate.astype(np.float32), T, C)
    hy = out.hybrid
    assert hy.n_dense_host() == pk.n_dense > 0
    np.testing.assert_array_equal(hy.counts.cpu().numpy(), pk.counts)
    np.testing.assert_array_equal(hy.indices.cpu().numpy(), pk.indices)
    np.testing.assert_array_equal(hy.dense_rows[:pk.n_dense].cpu().numpy(), pk.dense_rows)
    # values: h exact (stored zeros where the up branch is 0)
    np.testing.assert_array_equal(as_f64(twell.twell_unpack(hy)), h_ref)
    want = torch.from_numpy(y_ref).to(dtype)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out.y.cpu().view(bits), want.view(bits))


def test_gated_closed_gate_and_zero_rows():
    say("gated closed gate, 0 rows")
    cfg = synth.FfnConfig("gated", 100, 256, 1024, 128, 4, "bf16", -1.645)
    t = synth.make_gated_inputs(cfg)
    t["b_gate"] = torch.full((1024,), -1e4)
    out = run(t, 128, 4)
    assert int(out.status.item()) == twell.TWELL_OK and out.hybrid.n_dense_host() == 0
    assert not out.y.float().any()
    t0 = {k: (v[:0] if k == "x" else v) for k, v in t.items()}
    out0 = run(t0, 128, 4)
    assert out0.y.shape == (0, 256) and out0.hybrid.n_dense_host() == 0


@pytest.mark.parametrize("name", ["ffn_1b_bf16", "decode_bf16"])
def test_gated_full_size_sampled_rows(name):
    cfg = synth.CONFIGS[name]
    say(f"gated full size {name}")
    t = synth.make_gated_inputs(cfg)
    out = run(t, cfg.tile, cfg.capacity)
    assert int(out.status.item()) == twell.TWELL_OK
    rng = np.random.default_rng(5)
    nd = out.hybrid.n_dense_host()
    rows = np.unique(np.concatenate([rng.integers(0, cfg.n_rows, 24), [0, cfg.n_rows - 1],
                                     out.hybrid.dense_rows[:min(nd, 4)].cpu().numpy()]))
    sub = {k: (v[rows] if k == "x" else v) for k, v in t.items()}
    _, y_ref = ref(sub)
    assert_close_rel(as_f64(out.y)[rows], y_ref, TOL[cfg.torch_dtype], "y rows")
