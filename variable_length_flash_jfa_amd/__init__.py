"""MI355X (gfx950) Jagged Flash Attention.

Thin Python binding over the C ABI of ``_lib/libjfa.so`` (declared in
``include/jfa.h``).  Every step of the computation runs in the library's HIP
kernels; this package only marshals torch tensors, streams and workspaces.
"""
from ._binding import (  # noqa: F401
    JfaError,
    SCHED_SORTED_ZIGZAG,
    SCHED_IDENTITY,
    SCHED_DYNAMIC,
    fwd,
    fwd_sparse,
    fwd_mxfp8,
    mxfp8_quantize_rows,
    mxfp8_quantize_v,
    mxfp8_v_blocks,
    bwd,
    fwd_workspace_size,
    bwd_workspace_size,
    set_schedule,
    profile_enable,
    profile_read,
    get_schedule,
    library,
    library_path,
    version,
)
from .autograd import jagged_attention  # noqa: F401
