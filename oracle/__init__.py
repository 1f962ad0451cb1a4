"""CPU oracle for the hybrid-TwELL ReLU FFN forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product path never does.
"""
from .twell_oracle import (  # noqa: F401
    Ell,
    Grads,
    Hybrid,
    bf16_bits_to_f32,
    ell_pack,
    ell_pack_textbook,
    ell_unpack,
    ffn_backward,
    ffn_backward_from_h,
    ffn_forward,
    ffn_forward_rows,
    ffn_hidden,
    gated_ffn_forward,
    gated_ffn_hidden,
    pack,
    pack_reference,
    sampled_dots,
    spmm,
    tile_counts,
    to_csr,
    unpack,
)
