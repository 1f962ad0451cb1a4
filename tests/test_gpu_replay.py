"""Stream ordering of ffn_sparse_forward.  Captured into a HIP graph, every
replay equals the eager call bit for bit, with eager work and
synchronisations between replays (at 16 rows the capture holds the split-K
path); queued back to back on shared buffers, calls do not overlap."""
import numpy as np
import pytest
import torch

from activation_sparse_transformer_amd import twell
from activation_sparse_transformer_amd.synth import CONFIGS, make_inputs
from gpu_helpers import as_f32, inputs_to_device, say, u32

pytestmark = pytest.mark.gpu


def snapshot(b):
    nd = b.hybrid.n_dense_host()
    return (u32(as_f32(b.y)), b.hybrid.counts.cpu().numpy(), b.hybrid.indices.cpu().numpy(),
            u32(as_f32(b.hybrid.values)), nd, b.hybrid.dense_rows[:nd].cpu().numpy(),
            u32(as_f32(b.hybrid.dense_values[:nd])), int(b.status.item()))


@pytest.mark.parametrize("name,n,dm,dff", [("decode_bf16", 16, 512, 2048),
                                           ("ffn_1b_bf16", 300, 256, 1024),
                                           ("tiny_fp32", 64, 128, 512)])
def test_graph_replays_match_eager(name, n, dm, dff):
    say(f"graph capture {name} n={n}")
    cfg = CONFIGS[name].replace(n_rows=n, d_model=dm, d_ff=dff)
    d = inputs_to_device(make_inputs(cfg))
    bufs = twell.forward_buffers(cfg.n_rows, cfg.d_model, cfg.d_ff, cfg.tile, cfg.capacity,
                                 cfg.torch_dtype, torch.device("cuda:0"))
    run = lambda: twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"], cfg.tile,
                                           cfg.capacity, out=bufs)
    run()  # eager reference
    torch.cuda.synchronize()
    ref = snapshot(bufs)
    assert 0 < ref[4] < n or name == "tiny_fp32"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        bufs.y.fill_(7)  # eager work on the outputs between replays
        bufs.hybrid.counts.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(bufs)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)
    del g


def test_back_to_back_calls_on_shared_buffers():
    """Forward calls queued back to back on one stream, alternating two inputs
    and reusing the same output and workspace buffers, with no host
    synchronisation in between: each call must finish with the buffers before
    the next call reuses them.  The final outputs equal a lone call's, bit for
    bit."""
    cfg = CONFIGS["ffn_1b_bf16"].replace(n_rows=600, d_model=512, d_ff=2048)
    da = inputs_to_device(make_inputs(cfg))
    db = inputs_to_device(make_inputs(cfg.replace(seed=1)))
    bufs = twell.forward_buffers(cfg.n_rows, cfg.d_model, cfg.d_ff, cfg.tile, cfg.capacity,
                                 cfg.torch_dtype, torch.device("cuda:0"))
    run = lambda d: twell.ffn_sparse_forward(d["x"], d["w_up_t"], d["b_up"], d["w_down"],
                                             cfg.tile, cfg.capacity, out=bufs)
    refs = {}
    for name, d in (("a", da), ("b", db)):
        run(d)
        torch.cuda.synchronize()
        refs[name] = snapshot(bufs)
    assert not np.array_equal(refs["a"][0], refs["b"][0])
    for last in ("a", "b"):
        for i in range(40):
            run(db if (i % 2 == 0) == (last == "a") else da)
        run(da if last == "a" else db)
        torch.cuda.synchronize()
        got = snapshot(bufs)
        for x, y in zip(got, refs[last]):
            np.testing.assert_array_equal(x, y)
