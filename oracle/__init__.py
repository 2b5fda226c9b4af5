"""Plain fp64 CPU oracle for jagged flash attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it.
"""
from .attention import (  # noqa: F401
    sequence_forward,
    sequence_backward,
    sequence_dq_rows,
    forward,
    backward,
    row_count,
)
from .rope import rope_rotate, rope_conjugate, backward_rope  # noqa: F401
from . import sparse  # noqa: F401  (block-sparse top-k forward)
from . import mxfp8  # noqa: F401  (block-scaled 8-bit forward)
