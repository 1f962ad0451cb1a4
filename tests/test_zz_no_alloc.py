"""twell_pack_noalloc, the entry point that takes no workspace and allocates
nothing: through the C ABI it gives the same hybrid as twell_pack, bit for
bit, on two calls in a row (the second smaller, with another tile width and
capacity, on the same fixed device scratch), and it refuses a shape whose
workspace exceeds the scratch before enqueuing anything."""
import numpy as np
import pytest
import torch

from activation_sparse_transformer_amd import twell
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def sparse_h(seed, n, dff, density):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn((n, dff), generator=g).abs() + 0.01
    h[torch.rand((n, dff), generator=g) >= density] = 0
    return h.to(torch.bfloat16).cuda()


def same_hybrid(a, sa, b, sb):
    torch.cuda.synchronize()
    assert int(sa.item()) == int(sb.item()) == twell.TWELL_OK
    nd = a.n_dense_host()
    assert nd == b.n_dense_host() and 0 < nd < a.n_rows
    assert torch.equal(a.counts, b.counts)
    assert torch.equal(a.indices, b.indices)
    assert torch.equal(a.values.view(torch.int16), b.values.view(torch.int16))
    assert torch.equal(a.dense_rows[:nd], b.dense_rows[:nd])
    assert torch.equal(a.dense_values[:nd].view(torch.int16), b.dense_values[:nd].view(torch.int16))


def test_noalloc_pack_matches_pack_twice():
    cases = [(3000, 8192, 128, 4, 0.012), (700, 2048, 256, 8, 0.03)]  # the second smaller
    for n, dff, T, C, dens in cases:
        say(f"noalloc pack n={n} dff={dff} T={T} C={C}")
        h = sparse_h(n + dff, n, dff, dens)
        shape = twell.make_shape(n, 8, dff, T, C, torch.bfloat16)
        assert twell.pack_workspace_bytes(shape) <= twell.NOALLOC_SCRATCH_BYTES
        ref, sref = twell.twell_pack(h, T, C)
        got, sgot = twell.twell_pack_noalloc(h, T, C)
        same_hybrid(got, sgot, ref, sref)


def test_noalloc_pack_refuses_a_shape_beyond_its_scratch():
    # 1024 tiles of 64 per row x 16384 rows: 16 MiB of tile flags alone
    n, dff, T = 16384, 65536, 64
    shape = twell.make_shape(n, 8, dff, T, 1, torch.bfloat16)
    assert twell.pack_workspace_bytes(shape) > twell.NOALLOC_SCRATCH_BYTES
    h = torch.zeros((n, dff), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(twell.TwellError) as e:
        twell.twell_pack_noalloc(h, T, 1, dense_capacity=1)
    assert e.value.code == twell.TWELL_ERR_SCRATCH_LIMIT
