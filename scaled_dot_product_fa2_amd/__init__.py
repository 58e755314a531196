"""MI355X (gfx950) fused attention forward and backward.

The computation runs in the HIP library ``libfa.so`` (C ABI in include/fa.h);
this package only marshals arguments to it. PyTorch is used for device memory,
strides and the current stream. There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from ._binding import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_NOALLOC_MAX_ROWS, FaBwdCall, FaCall, FaError, fa_bwd, fa_bwd_call,
                       fa_bwd_noalloc, fa_bwd_varlen, fa_fwd, fa_fwd_balance_applies, fa_fwd_call, fa_fwd_plan,
                       fa_fwd_varlen, fa_fwd_window, fa_strerror, fa_tile_pairs, fa_version, lib_path, load_library)

__all__ = ["fa_fwd", "fa_fwd_window", "fa_fwd_varlen", "fa_bwd", "fa_bwd_varlen", "fa_bwd_noalloc", "fa_fwd_call", "FaCall",
           "fa_bwd_call", "FaBwdCall", "fa_fwd_balance_applies",
           "fa_fwd_plan", "fa_tile_pairs", "fa_strerror", "fa_version", "FaError", "FA_DTYPE_F16", "FA_DTYPE_BF16",
           "FA_NOALLOC_MAX_ROWS",
           "lib_path", "load_library"]
