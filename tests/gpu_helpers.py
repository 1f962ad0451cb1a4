"""Helpers for the GPU parity tests: move GPU results to the oracle's terms
and compare them.  Nothing here computes the method; it only converts and
compares."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from activation_sparse_transformer_amd import twell

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def as_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 numpy copy of an fp32 / bf16 tensor."""
    return t.detach().float().cpu().numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().double().cpu().numpy()


def u32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def gpu_hybrid_rows(hy: twell.Hybrid, rows=None):
    """TwELL arrays of a GPU hybrid (optionally a subset of rows) on the host."""
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=hy.counts.device)
    return (as_f32(hy.values[sel]), hy.indices[sel].cpu().numpy(), hy.counts[sel].cpu().numpy())


def assert_pack_matches(hy: twell.Hybrid, h_host: np.ndarray, check_dense_values: bool = True):
    """Bit-exact comparison of a GPU hybrid with the oracle's pack of h_host
    (float32 holding the exact storage-dtype values)."""
    ref = oracle.pack(h_host, hy.tile, hy.capacity)
    vals, idx, cnt = gpu_hybrid_rows(hy)
    np.testing.assert_array_equal(cnt, ref.counts)
    np.testing.assert_array_equal(idx, ref.indices)
    np.testing.assert_array_equal(u32(vals), u32(ref.values))
    n_dense = hy.n_dense_host()
    assert n_dense == ref.n_dense, (n_dense, ref.n_dense)
    stored = min(n_dense, hy.dense_capacity)
    np.testing.assert_array_equal(hy.dense_rows[:stored].cpu().numpy(), ref.dense_rows[:stored])
    if check_dense_values and stored:
        np.testing.assert_array_equal(u32(as_f32(hy.dense_values[:stored])),
                                      u32(ref.dense_values[:stored]))
    return ref


def assert_close_rel(got: np.ndarray, ref: np.ndarray, tol: float, what: str = "y"):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if ref.size else 0.0
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol} * max|ref| {scale:.3e}"
    return err, scale


def inputs_to_device(t: dict, device="cuda"):
    return {k: v.to(device) for k, v in t.items()}


def oracle_inputs(t: dict):
    return (t["x"].double().numpy(), t["w_up_t"].double().numpy(), t["b_up"].double().numpy(),
            t["w_down"].double().numpy())
