"""Sparse top-k MLA attention (prefill and paged decode forward, prefill
backward) and block-sparse MLA attention forward for MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of include/sparse_mla.h (libsparse_mla.so); this package only binds it.
"""
from ._binding import (EXPORTS, SparseMLAError, block_sparse_fwd, bwd,  # noqa: F401
                       bwd_workspace_bytes, decode_fwd, decode_fwd_split,
                       decode_fwd_split_noalloc, decode_num_splits,
                       decode_split_noalloc_max_bytes, decode_split_workspace_bytes, fwd,
                       last_kernel, load_library, row_lengths)

__all__ = ["fwd", "bwd", "block_sparse_fwd", "bwd_workspace_bytes", "decode_fwd",
           "decode_fwd_split", "decode_fwd_split_noalloc", "decode_num_splits",
           "decode_split_noalloc_max_bytes", "decode_split_workspace_bytes", "row_lengths",
           "last_kernel", "load_library", "SparseMLAError", "EXPORTS"]
