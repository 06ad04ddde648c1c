"""Sparse top-k MLA attention forward (prefill and paged decode) for MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of include/sparse_mla.h (libsparse_mla.so); this package only binds it.
"""
from ._binding import (EXPORTS, SparseMLAError, decode_fwd, fwd, load_library,  # noqa: F401
                       row_lengths)

__all__ = ["fwd", "decode_fwd", "row_lengths", "load_library", "SparseMLAError", "EXPORTS"]
