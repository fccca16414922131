"""Parallax attention (parameterized Local Linear Attention) for AMD MI355X.

The compute path is the HIP library ``libplx.so`` (C ABI in ``include/plx.h``);
this package only loads it and marshals torch tensors into its calls.
"""

from .binding import (  # noqa: F401
    PLX_NO_INTERCEPT,
    PLX_UNIFORM_WEIGHTS,
    PlxError,
    bwd_workspace_size,
    decode_workspace_size,
    lib,
    plx_bwd,
    plx_decode,
    plx_decode_ex,
    plx_decode_noalloc,
    plx_fwd_prefill,
    plx_fwd_prefill_ex,
    plx_qkvr_proj,
    status_string,
)
