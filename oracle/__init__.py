"""CPU fp64 oracle for token-level dynamic local-global attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers allowed. The product (the HIP library
and its Python binding) never imports it, and it imports nothing from the
product. See ``oracle/logo.py`` for the definition it computes and the
passages each step follows.

Parity status: every function here is pinned (tests/test_oracle.py); none is
"parity unpinned" against the mathematics, though the pages themselves print
no worked numbers for this method.
"""
from .logo import (  # noqa: F401
    combine,
    default_scale,
    forward,
    forward_rows,
    global_attention,
    global_row,
    local_attention,
    local_row,
    select_queries,
    sigmoid,
    softmax_weights,
    target_count,
)
