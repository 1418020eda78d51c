"""CPU fp64 oracle for token-level dynamic local-global attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers allowed. The product (the HIP library
and its Python binding) never imports it, and it imports nothing from the
product. See ``oracle/logo.py`` for the forward's definition and the passages
each step follows, and ``oracle/backward.py`` for its chain rule (gradients
of q, k, v and the gate, and the statistics a training forward saves), and
``oracle/router.py`` for the routed forward (the gate computed from the local
branch's output), and ``oracle/decode.py`` for the threshold budget
controller and the decode step, and ``oracle/varlen.py`` for packed
variable-length batches.

Parity status: every function here is pinned (tests/test_oracle.py,
tests/test_oracle_backward.py, tests/test_oracle_router.py, tests/test_oracle_decode.py, tests/test_oracle_varlen.py);
none is
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
from . import backward  # noqa: F401,E402
from . import router  # noqa: F401,E402
from . import decode  # noqa: F401,E402
from . import varlen  # noqa: F401,E402
