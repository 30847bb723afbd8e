"""Exact tiled attention for MI355X (gfx950).

Python binding of libfa.so: the functions below carry the C-ABI names of
``include/fa.h`` and only marshal arguments (device pointers, sizes, the
current HIP stream).  Every step of the computation runs in the library's HIP
kernels; there is no other code path.  If libfa.so has not been built,
importing the binding raises.
"""
from ._binding import (  # noqa: F401
    FAError,
    FA_DTYPE_BF16,
    FA_DTYPE_F16,
    FA_DECODE_MAX_Q,
    FA_MASK_BLOCK,
    FA_MASK_MAX_N,
    FA_NOALLOC_MAX_ROWS,
    fa_backward,
    fa_backward_keep,
    fa_backward_keep_stage,
    fa_backward_noalloc,
    fa_backward_stage,
    fa_backward_workspace_size,
    fa_decode,
    fa_decode_paged,
    fa_decode_workspace_size,
    fa_dropout_bits_size,
    fa_dropout_mask,
    fa_forward,
    fa_forward_keep,
    fa_strerror,
    library_path,
)

__all__ = [
    "FAError", "FA_DTYPE_BF16", "FA_DTYPE_F16", "FA_DECODE_MAX_Q", "FA_MASK_BLOCK", "FA_MASK_MAX_N", "FA_NOALLOC_MAX_ROWS", "fa_backward", "fa_backward_keep",
    "fa_backward_keep_stage", "fa_backward_noalloc", "fa_backward_stage", "fa_backward_workspace_size", "fa_decode", "fa_decode_paged", "fa_decode_workspace_size", "fa_dropout_bits_size", "fa_dropout_mask", "fa_forward", "fa_forward_keep",
    "fa_strerror", "library_path",
]
