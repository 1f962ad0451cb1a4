"""Seeded synthetic inputs for the ReLU-sparse FFN layer.

This module only draws random numbers and casts them to the storage dtype.
It holds none of the method's arithmetic (no GEMM, no ReLU, no packing), so
both the CPU oracle's tests and the HIP path's tests and benchmark can take
their inputs from here without sharing any of the computation under test.

Workloads: the pages measure billion-parameter ReLU-sparse models on H100
("Nvidia and Sakana make LLMs 30% faster by doing less math", section
"More speed, less power, zero quality loss") with no trained weights or data
available here, so seeded Gaussian FFN layers of the same role stand in:

* x ~ N(0, 1), optionally scaled per token by a log-normal factor;
* W_up ~ N(0, 1/d_model), stored transposed as ``w_up_t[d_ff, d_model]``;
* W_down ~ N(0, 1/d_ff), stored as ``w_down[d_ff, d_model]``;
* b_up = b0 (+ per-neuron Gaussian noise), kept in fp32.

Every "N(0, s)" and "LogNormal(0, s)" parameter is read as a variance: with
x ~ N(0, 1) and W_up ~ N(0, 1/d_model) the pre-activation is ~N(b0, 1), so
b0 = -1.645 / -2.326 / -1.282 gives the stated ~5% / ~1% / ~10% active units
only under that reading.

Random stream layout (fixed, independent of thread count): one
``SeedSequence(seed)`` spawns seven children [x, token-scale, W_up, bias-noise,
W_down, dy, W_up of a gated layer's up branch] (dy: the upstream gradient of
the backward pass, ~N(0, 1); the gated layer takes the plain recipe's W_up and
b as its gate and draws its up branch ~N(0, 1/d_model), bias 0); each tensor's child spawns one grandchild per block of
``CHUNK_ROWS`` rows, and each block is drawn with
``Generator(PCG64(grandchild)).standard_normal(..., dtype=float32)`` in
row-major order.  Blocks are drawn on a thread pool.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from numpy.random import PCG64, Generator, SeedSequence

CHUNK_ROWS = 256

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class FfnConfig:
    """One synthetic FFN layer: shapes, TwELL geometry and input recipe."""

    name: str
    n_rows: int  # tokens N
    d_model: int
    d_ff: int
    tile: int  # TwELL tile width T
    capacity: int  # TwELL slots per tile C
    dtype: str  # "fp32" or "bf16": storage dtype of x, W, h and y
    b0: float  # up-projection bias
    token_scale_var: float = 0.0  # variance of log of per-token x scale (0: none)
    bias_noise_var: float = 0.0  # variance of per-neuron bias noise (0: none)
    seed: int = 0

    @property
    def n_tiles(self) -> int:
        return self.d_ff // self.tile

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def replace(self, **kw) -> "FfnConfig":
        return dataclasses.replace(self, **kw)


# The five layers the benchmark and the parity tests use.
CONFIGS = {
    "tiny_fp32": FfnConfig("tiny_fp32", 64, 128, 512, 64, 8, "fp32", -1.645),
    "ffn_1b_bf16": FfnConfig("ffn_1b_bf16", 4096, 2048, 8192, 128, 4, "bf16", -2.326),
    "hybrid_stress_bf16": FfnConfig(
        "hybrid_stress_bf16", 8192, 4096, 14336, 128, 4, "bf16", -2.326,
        token_scale_var=0.5, bias_noise_var=0.2),
    "decode_bf16": FfnConfig("decode_bf16", 16, 4096, 16384, 128, 4, "bf16", -2.326),
    "large_bf16": FfnConfig(
        "large_bf16", 16384, 8192, 28672, 256, 8, "bf16", -1.282,
        token_scale_var=0.5),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_normal(seq: SeedSequence, shape: tuple[int, int]) -> np.ndarray:
    """Standard normals [rows, cols] float32 under the fixed block layout."""
    rows, cols = shape
    nblk = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    out = np.empty((rows, cols), dtype=np.float32)
    kids = seq.spawn(nblk) if nblk else []

    def fill(i: int) -> None:
        r0 = i * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        Generator(PCG64(kids[i])).standard_normal(
            (r1 - r0, cols), dtype=np.float32, out=out[r0:r1])

    if nblk > 1:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nblk)))
    elif nblk == 1:
        fill(0)
    return out


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DTYPES[dtype])  # torch's CPU cast to bf16 rounds to nearest even


def make_inputs(cfg: FfnConfig) -> dict[str, torch.Tensor]:
    """Return CPU tensors x [N,dm], w_up_t [dff,dm], b_up [dff] fp32, w_down [dff,dm]."""
    s_x, s_scale, s_wup, s_bnoise, s_wdown = SeedSequence(cfg.seed).spawn(5)
    n, dm, dff = cfg.n_rows, cfg.d_model, cfg.d_ff

    x = draw_normal(s_x, (n, dm))
    if cfg.token_scale_var > 0 and n > 0:
        u = draw_normal(s_scale, (1, n))[0].astype(np.float64)
        scale = np.exp(math.sqrt(cfg.token_scale_var) * u).astype(np.float32)
        x *= scale[:, None]

    w_up_t = draw_normal(s_wup, (dff, dm))
    w_up_t *= np.float32(1.0 / math.sqrt(dm))

    b = np.full(dff, cfg.b0, dtype=np.float64)
    if cfg.bias_noise_var > 0:
        b += math.sqrt(cfg.bias_noise_var) * draw_normal(s_bnoise, (1, dff))[0]

    w_down = draw_normal(s_wdown, (dff, dm))
    w_down *= np.float32(1.0 / math.sqrt(dff))

    return {
        "x": _cast(x, cfg.dtype),
        "w_up_t": _cast(w_up_t, cfg.dtype),
        "b_up": torch.from_numpy(b.astype(np.float32)),
        "w_down": _cast(w_down, cfg.dtype),
    }


def make_grad(cfg: FfnConfig) -> torch.Tensor:
    """Return dy [N, d_model] ~ N(0, 1) in the storage dtype (CPU): the
    upstream gradient of the layer's output, from the sixth child stream."""
    s_dy = SeedSequence(cfg.seed).spawn(6)[5]
    return _cast(draw_normal(s_dy, (cfg.n_rows, cfg.d_model)), cfg.dtype)


def make_gated_inputs(cfg: FfnConfig) -> dict[str, torch.Tensor]:
    """Inputs of the ReLU-gated layer: x, w_gate_t / b_gate (the plain
    recipe's W_up and b, so the gate has the plain layer's sparsity), w_up_t
    ~N(0, 1/d_model) from the seventh child stream, b_up = 0 (fp32), w_down."""
    t = make_inputs(cfg)
    s_up = SeedSequence(cfg.seed).spawn(7)[6]
    w = draw_normal(s_up, (cfg.d_ff, cfg.d_model))
    w *= np.float32(1.0 / math.sqrt(cfg.d_model))
    return {"x": t["x"], "w_gate_t": t["w_up_t"], "b_gate": t["b_up"], "w_up_t": _cast(w, cfg.dtype),
            "b_up": torch.zeros(cfg.d_ff, dtype=torch.float32), "w_down": t["w_down"]}

