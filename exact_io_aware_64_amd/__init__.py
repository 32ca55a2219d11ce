"""Exact, IO-aware, tiled attention for MI355X (gfx950).

The computation lives in libfa.so (HIP kernels behind the C ABI of
include/fa.h); this package only builds and binds it.  Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    FA_BF16,
    FA_F32,
    FaError,
    backward,
    bwd,
    fa_bwd,
    fa_bwd_dkdv,
    fa_bwd_noalloc,
    fa_bwd_dq,
    fa_bwd_qk,
    fa_bwd_dropout,
    fa_bwd_workspace_bytes,
    fa_fwd,
    fa_fwd_dropout,
    fa_fwd_key_groups,
    fa_fwd_qk,
    fa_fwd_tiled,
    fa_last_error,
    fa_status_string,
    forward,
    fwd,
    load_library,
    prepare_bwd,
    prepare_fwd,
    prepare_fwd_tiled,
)
