"""CPU oracle for one tensor-parallel rank's share of a transformer block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package; only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (``tensor_transformer_linear_tp_amd``) and does not import it.

Everything here is plain float64 numpy: library matmul / sum / exp / erf are
the only primitives, with no blocking, fusion or reordering beyond the
definitions the pages state.  Its own pins live in ``tests/test_oracle_*.py``.
"""
from .tp_oracle import (  # noqa: F401
    column_slice,
    row_slice,
    gelu,
    gelu_grad,
    silu,
    silu_grad,
    sigmoid,
    column_fwd,
    row_fwd,
    sum_partials,
    act_bwd,
    row_bwd,
    column_bwd,
    dgrad,
    wgrad,
    vocab_ce_partials,
    lse_recombine,
    vocab_ce_bwd,
    layer_norm,
    sp_reduce_scatter_ln,
    vocab_embed_fwd,
    vocab_embed_bwd,
    attention_fwd,
    attention_bwd,
)
