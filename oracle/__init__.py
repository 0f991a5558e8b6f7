"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE: imported only by the test suite, the smoke check and the
bench's CPU-baseline leg. The GPU library does not import it and it imports
nothing from the GPU library.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    attn_bwd,
    attn_fwd_naive,
    attn_fwd_tiled,
    block_state,
    finalize,
    merge,
    online_row,
    softmax_row_output,
    visible,
)
