"""GPU parity of the ELL rows (Figure 1(a) with the hybrid split) against the
CPU oracle: ell_pack bit-exact (slots, columns, counts, dense-row list, dense
rows) against the oracle's ELL packer on the same h; ell_unpack(ell_pack(h))
equal to h bitwise; ell_spmm exact on integer-valued data (every product
and partial sum an integer below 2^8), through the XCD-sliced list kernel
(bf16, d_model a multiple of 512) and the per-chunk kernel."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_transformer_amd import twell
from gpu_helpers import as_f32, as_f64, say, u32

pytestmark = pytest.mark.gpu
DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def sparse_h(seed, n, dff, density, dtype, negzero=False, nan=False):
    rng = np.random.default_rng(seed)
    h = np.abs(rng.standard_normal((n, dff))).astype(np.float32) + 0.01
    h *= np.where(rng.random((n, dff)) < 0.5, 1, -1).astype(np.float32)
    h[rng.random((n, dff)) >= density] = 0.0
    if negzero:
        z = np.argwhere(h == 0)[::5]
        h[z[:, 0], z[:, 1]] = -0.0
    if nan and n:
        h[rng.integers(0, n, 3), rng.integers(0, dff, 3)] = np.nan
    t = torch.from_numpy(h).to(dtype)
    return t, as_f32(t)


def assert_ell_matches(e: twell.Ell, h_host: np.ndarray, check_dense_values=True):
    ref = oracle.ell_pack(h_host, e.width)
    n = h_host.shape[0]
    cnt = e.counts.cpu().numpy().view(np.uint16).astype(np.int64)
    cols = e.columns.cpu().numpy().view(np.uint16).astype(np.int64)
    np.testing.assert_array_equal(cnt, ref.counts)
    np.testing.assert_array_equal(cols, ref.columns)
    np.testing.assert_array_equal(u32(as_f32(e.values)), u32(ref.values))
    nd = e.n_dense_host()
    assert nd == ref.n_dense, (nd, ref.n_dense)
    stored = min(nd, e.dense_capacity)
    np.testing.assert_array_equal(e.dense_rows[:stored].cpu().numpy(), ref.dense_rows[:stored])
    if check_dense_values and stored:
        np.testing.assert_array_equal(u32(as_f32(e.dense_values[:stored])),
                                      u32(ref.dense_values[:stored]))
    assert n == 0 or cnt.max() <= e.width
    return ref


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,dff,width,density", [(1, 256, 4, 0.02), (77, 640, 8, 0.01),
                                                 (300, 1024, 12, 0.01), (1500, 512, 6, 0.01),
                                                 (64, 2048, 256, 0.1)])
def test_ell_pack_bitexact_and_round_trip(dtype, n, dff, width, density):
    say(f"ell pack {dtype} n={n} dff={dff} width={width}")
    ht, hh = sparse_h(n + dff + width, n, dff, density, DT[dtype], negzero=True, nan=(n == 300))
    e, status = twell.ell_pack(ht.cuda(), width)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_OK
    ref = assert_ell_matches(e, hh)
    if n > 1:
        assert 0 < ref.n_dense < n or width == 256
    u = twell.ell_unpack(e)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u32(as_f32(u)), u32(oracle.ell_unpack(ref)))


def test_ell_round_trip_bitwise_on_relu_output():
    """h as a ReLU writes it (+0.0 for inactive units): unpack(pack(h)) == h."""
    g = torch.Generator().manual_seed(3)
    h = torch.relu(torch.randn((700, 2048), generator=g) - 2.3).to(torch.bfloat16).cuda()
    e, _ = twell.ell_pack(h, 24)
    u = twell.ell_unpack(e)
    torch.cuda.synchronize()
    assert 0 < e.n_dense_host() < 700
    assert torch.equal(u.view(torch.int16), h.view(torch.int16))


def test_ell_dense_capacity_exceeded_and_zero_rows():
    ht, hh = sparse_h(5, 200, 512, 0.02, torch.bfloat16)
    ref = oracle.ell_pack(hh, 6)
    assert ref.n_dense > 10
    e, status = twell.ell_pack(ht.cuda(), 6, dense_capacity=10)
    torch.cuda.synchronize()
    assert int(status.item()) == twell.TWELL_ERR_DENSE_CAPACITY
    assert e.n_dense_host() == ref.n_dense
    np.testing.assert_array_equal(e.dense_rows.cpu().numpy(), ref.dense_rows[:10])
    np.testing.assert_array_equal(e.counts.cpu().numpy().view(np.uint16), ref.counts)
    h0 = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    e0, s0 = twell.ell_pack(h0, 4)
    torch.cuda.synchronize()
    assert int(s0.item()) == 0 and e0.n_dense_host() == 0
    assert twell.ell_unpack(e0).shape == (0, 256)


@pytest.mark.parametrize("dtype,n,dm,dff,width", [("bf16", 300, 2048, 1024, 10),
                                                  ("bf16", 1500, 512, 2048, 20),
                                                  ("bf16", 200, 136, 640, 8),
                                                  ("fp32", 300, 520, 1024, 10),
                                                  ("fp32", 70, 64, 768, 6)])
def test_ell_spmm_integer_exact(dtype, n, dm, dff, width):
    say(f"ell spmm {dtype} n={n} dm={dm} dff={dff} width={width}")
    rng = np.random.default_rng(n + dm + dff)
    h = rng.integers(-2, 3, size=(n, dff)).astype(np.float32)
    h[rng.random((n, dff)) >= 0.01] = 0
    w = rng.integers(-1, 2, size=(dff, dm)).astype(np.float32)
    w[rng.random((dff, dm)) < 0.7] = 0
    ht = torch.from_numpy(h).to(DT[dtype]).cuda()
    e, _ = twell.ell_pack(ht, width)
    y = torch.full((n, dm), float("nan"), dtype=DT[dtype], device="cuda")
    twell.ell_spmm(e, torch.from_numpy(w).to(DT[dtype]).cuda(), out=y)
    torch.cuda.synchronize()
    ref = assert_ell_matches(e, h)
    assert 0 < ref.n_dense < n
    y_ref = h.astype(np.float64) @ w.astype(np.float64)  # the plain definition
    assert np.max(np.abs(y_ref)) <= 256
    np.testing.assert_array_equal(as_f64(y), y_ref)   # every row written, no NaN left
