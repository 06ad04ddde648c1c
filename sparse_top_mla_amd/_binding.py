"""ctypes binding of libsparse_mla.so (the C ABI in include/sparse_mla.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current HIP
stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIBRARY = _PKG / "libsparse_mla.so"

_STATUS = {0: "SMLA_OK", 1: "SMLA_ERR_NULL_ARG", 2: "SMLA_ERR_BAD_SHAPE", 3: "SMLA_ERR_UNSUPPORTED",
           4: "SMLA_ERR_LAUNCH"}

EXPORTS = ("sparse_mla_fwd", "sparse_mla_decode_fwd", "sparse_mla_decode_split_workspace_bytes",
           "sparse_mla_decode_fwd_split", "sparse_mla_decode_split_noalloc_max_bytes",
           "sparse_mla_decode_fwd_split_noalloc", "sparse_mla_row_lengths",
           "sparse_mla_bwd_workspace_bytes", "sparse_mla_bwd", "sparse_mla_block_sparse_fwd",
           "sparse_mla_last_error", "sparse_mla_last_kernel")

_lib = None


class SparseMLAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load_library(path: Path | None = None):
    """Load the HIP library (no GPU needed to load it).  Raises if absent."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(str(path)))
    if _lib is None:
        if not LIBRARY.exists():
            raise RuntimeError(f"{LIBRARY} is not built; run __graft_entry__.build() "
                               "(or python -m sparse_top_mla_amd.build)")
        _lib = _declare(ctypes.CDLL(str(LIBRARY)))
    return _lib


def _declare(lib):
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.sparse_mla_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                   vp, vp, vp, vp]
    lib.sparse_mla_fwd.restype = ctypes.c_int
    lib.sparse_mla_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, i32, f32, vp, vp, vp, vp]
    lib.sparse_mla_decode_fwd.restype = ctypes.c_int
    lib.sparse_mla_decode_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sparse_mla_decode_split_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse_mla_decode_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                i32, i32, i32, i32, i32, f32, i32, vp,
                                                ctypes.c_size_t, vp, vp, vp, vp]
    lib.sparse_mla_decode_fwd_split.restype = ctypes.c_int
    lib.sparse_mla_decode_split_noalloc_max_bytes.argtypes = []
    lib.sparse_mla_decode_split_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.sparse_mla_decode_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                        i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                                        vp, vp, vp, vp]
    lib.sparse_mla_decode_fwd_split_noalloc.restype = ctypes.c_int
    lib.sparse_mla_row_lengths.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.sparse_mla_row_lengths.restype = ctypes.c_int
    lib.sparse_mla_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sparse_mla_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse_mla_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                   f32, i32, vp, ctypes.c_size_t, vp, vp, vp, vp]
    lib.sparse_mla_bwd.restype = ctypes.c_int
    lib.sparse_mla_block_sparse_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                i32, i32, f32, vp, vp, vp]
    lib.sparse_mla_block_sparse_fwd.restype = ctypes.c_int
    lib.sparse_mla_last_error.argtypes = []
    lib.sparse_mla_last_error.restype = ctypes.c_char_p
    lib.sparse_mla_last_kernel.argtypes = []
    lib.sparse_mla_last_kernel.restype = ctypes.c_char_p
    return lib


def _check(lib, status):
    if status != 0:
        raise SparseMLAError(status, lib.sparse_mla_last_error().decode())


def _dev(t, name, dtype, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def fwd(q, kv, indices, sm_scale, d_v=512, attn_sink=None, topk_length=None, *, out=None,
        lse=None, max_logits=None, stream=None):
    """Sparse prefill forward.  q [s_q, h_q, d_qk] bf16, kv [s_kv, 1, d_qk]
    bf16, indices [s_q, 1, topk] int32, topk_length [s_q] int32 or None,
    attn_sink [h_q] fp32 or None.  Returns (out, lse, max_logits)."""
    lib = load_library()
    dev = q.device
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16, dev)
    _dev(indices, "indices", torch.int32, dev)
    _dev(topk_length, "topk_length", torch.int32, dev)
    _dev(attn_sink, "attn_sink", torch.float32, dev)
    if q.dim() != 3 or kv.dim() != 3 or indices.dim() != 3:
        raise ValueError("q, kv and indices must be 3-d ([s_q,h_q,d_qk], [s_kv,h_kv,d_qk], [s_q,h_kv,topk])")
    s_q, h_q, d_qk = q.shape
    s_kv, h_kv = kv.shape[0], kv.shape[1]
    topk = indices.shape[-1]
    if kv.shape[2] != d_qk or indices.shape[0] != s_q or indices.shape[1] != h_kv:
        raise ValueError("inconsistent shapes of q, kv and indices")
    if topk_length is not None and tuple(topk_length.shape) != (s_q,):
        raise ValueError("topk_length must have shape [s_q]")
    if attn_sink is not None and tuple(attn_sink.shape) != (h_q,):
        raise ValueError("attn_sink must have shape [h_q]")
    out = torch.empty((s_q, h_q, d_v), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((s_q, h_q), dtype=torch.float32, device=dev) if lse is None else lse
    max_logits = torch.empty((s_q, h_q), dtype=torch.float32, device=dev) if max_logits is None else max_logits
    _dev(out, "out", torch.bfloat16, dev)
    _dev(lse, "lse", torch.float32, dev)
    _dev(max_logits, "max_logits", torch.float32, dev)
    if out.numel() != s_q * h_q * d_v or lse.numel() != s_q * h_q or max_logits.numel() != s_q * h_q:
        raise ValueError("output buffers have the wrong size")
    st = lib.sparse_mla_fwd(_p(q), _p(kv), _p(indices), _p(topk_length), _p(attn_sink), s_q, s_kv,
                            h_q, h_kv, d_qk, d_v, topk, float(sm_scale), _p(out), _p(lse),
                            _p(max_logits), _stream(dev, stream))
    _check(lib, st)
    return out, lse, max_logits


def _decode_prep(q, kv_cache, block_table, cache_seqlens, indices, d_v, attn_sink, topk_length,
                 out, lse, max_logits, return_max_logits=True):
    """Checks and output buffers shared by the decode entry points
    (max_logits stays None when return_max_logits is false and none is
    given: the library then stores none)."""
    dev = q.device
    _dev(q, "q", torch.bfloat16)
    _dev(kv_cache, "kv_cache", torch.bfloat16, dev)
    _dev(block_table, "block_table", torch.int32, dev)
    _dev(cache_seqlens, "cache_seqlens", torch.int32, dev)
    _dev(indices, "indices", torch.int32, dev)
    _dev(attn_sink, "attn_sink", torch.float32, dev)
    if q.dim() != 4 or kv_cache.dim() != 4 or indices.dim() != 3 or block_table.dim() != 2:
        raise ValueError("q [B,s_q,h_q,d_qk], kv_cache [blocks,page,h_kv,d_qk], indices [B,s_q,topk], "
                         "block_table [B,mbps] expected")
    B, s_q, h_q, d_qk = q.shape
    num_blocks, page_size, h_kv = kv_cache.shape[0], kv_cache.shape[1], kv_cache.shape[2]
    topk = indices.shape[-1]
    if (kv_cache.shape[3] != d_qk or tuple(indices.shape[:2]) != (B, s_q) or block_table.shape[0] != B
            or tuple(cache_seqlens.shape) != (B,)):
        raise ValueError("inconsistent decode shapes")
    if topk_length is not None:
        _dev(topk_length, "topk_length", torch.int32, dev)
        if tuple(topk_length.shape) == (B,):
            topk_length = topk_length.view(B, 1).expand(B, s_q).contiguous()
        elif tuple(topk_length.shape) != (B, s_q):
            raise ValueError("topk_length must have shape [B] or [B, s_q]")
    if attn_sink is not None and tuple(attn_sink.shape) != (h_q,):
        raise ValueError("attn_sink must have shape [h_q]")
    out = torch.empty((B, s_q, h_q, d_v), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev) if lse is None else lse
    if max_logits is None and return_max_logits:
        max_logits = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.bfloat16, dev)
    _dev(lse, "lse", torch.float32, dev)
    _dev(max_logits, "max_logits", torch.float32, dev)
    if (out.numel() != B * s_q * h_q * d_v or lse.numel() != B * s_q * h_q
            or (max_logits is not None and max_logits.numel() != B * s_q * h_q)):
        raise ValueError("output buffers have the wrong size")
    return (B, s_q, h_q, d_qk, num_blocks, page_size, h_kv, topk, topk_length, out, lse,
            max_logits)


def decode_fwd(q, kv_cache, block_table, cache_seqlens, indices, sm_scale, d_v=512,
               attn_sink=None, topk_length=None, *, out=None, lse=None, max_logits=None,
               return_max_logits=True, stream=None):
    """Paged sparse decode forward.  q [B, s_q, h_q, d_qk] bf16,
    kv_cache [num_blocks, page_size, 1, d_qk] bf16, block_table [B, mbps]
    int32, cache_seqlens [B] int32, indices [B, s_q, topk] int32,
    topk_length [B, s_q] (or [B], broadcast over s_q) int32 or None,
    attn_sink [h_q] fp32 or None.  Returns (out, lse, max_logits);
    max_logits is None (and not stored) with return_max_logits=False."""
    lib = load_library()
    dev = q.device
    (B, s_q, h_q, d_qk, num_blocks, page_size, h_kv, topk, topk_length, out, lse,
     max_logits) = _decode_prep(q, kv_cache, block_table, cache_seqlens, indices, d_v, attn_sink,
                                topk_length, out, lse, max_logits, return_max_logits)
    st = lib.sparse_mla_decode_fwd(_p(q), _p(kv_cache), _p(block_table), _p(cache_seqlens),
                                   _p(indices), _p(topk_length), _p(attn_sink), B, s_q, h_q, h_kv,
                                   d_qk, d_v, topk, num_blocks, page_size, block_table.shape[1],
                                   float(sm_scale), _p(out), _p(lse), _p(max_logits),
                                   _stream(dev, stream))
    _check(lib, st)
    return out, lse, max_logits


def decode_num_splits(B, s_q, topk, device=None):
    """A split count for decode_fwd_split: about four 64-key blocks per split,
    and no more (row, split) units than the device has CUs (measured on
    MI355X at B = 2, s_q = 2, topk = 2048: 8 splits, 40.7 us against 112 us
    unsplit; 4 to 16 splits are within 20%).  1 when the rows alone fill the
    device."""
    rows = B * s_q
    cus = torch.cuda.get_device_properties(device or 0).multi_processor_count
    if rows <= 0 or rows >= cus:
        return 1
    blocks = -(-topk // 64)
    return max(1, min(-(-blocks // 4), -(-cus // rows)))


def decode_split_workspace_bytes(B, s_q, h_q, d_v, num_splits):
    """Workspace bytes sparse_mla_decode_fwd_split needs."""
    return int(load_library().sparse_mla_decode_split_workspace_bytes(B, s_q, h_q, d_v, num_splits))


def decode_fwd_split(q, kv_cache, block_table, cache_seqlens, indices, sm_scale, num_splits,
                     d_v=512, attn_sink=None, topk_length=None, *, workspace=None, out=None,
                     lse=None, max_logits=None, return_max_logits=True, stream=None):
    """Split-KV paged decode: arguments and results as decode_fwd; each row's
    index blocks are split num_splits ways and merged.  `workspace` (a uint8
    CUDA tensor of at least decode_split_workspace_bytes(...) bytes) is
    allocated here when not given."""
    lib = load_library()
    dev = q.device
    (B, s_q, h_q, d_qk, num_blocks, page_size, h_kv, topk, topk_length, out, lse,
     max_logits) = _decode_prep(q, kv_cache, block_table, cache_seqlens, indices, d_v, attn_sink,
                                topk_length, out, lse, max_logits, return_max_logits)
    need = lib.sparse_mla_decode_split_workspace_bytes(B, s_q, h_q, d_v, int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, dev)
    st = lib.sparse_mla_decode_fwd_split(_p(q), _p(kv_cache), _p(block_table), _p(cache_seqlens),
                                         _p(indices), _p(topk_length), _p(attn_sink), B, s_q, h_q,
                                         h_kv, d_qk, d_v, topk, num_blocks, page_size,
                                         block_table.shape[1], float(sm_scale), int(num_splits),
                                         _p(workspace), workspace.numel(), _p(out), _p(lse),
                                         _p(max_logits), _stream(dev, stream))
    _check(lib, st)
    return out, lse, max_logits


def decode_split_noalloc_max_bytes():
    """Bytes of the static partials array of decode_fwd_split_noalloc."""
    return int(load_library().sparse_mla_decode_split_noalloc_max_bytes())


def decode_fwd_split_noalloc(q, kv_cache, block_table, cache_seqlens, indices, sm_scale,
                             num_splits, d_v=512, attn_sink=None, topk_length=None, *, out=None,
                             lse=None, max_logits=None, return_max_logits=True, stream=None):
    """Split-KV paged decode whose partials live in the library's static
    device array (the entry point allocates nothing; outputs are allocated
    here when not given).  Arguments and results as decode_fwd_split."""
    lib = load_library()
    dev = q.device
    (B, s_q, h_q, d_qk, num_blocks, page_size, h_kv, topk, topk_length, out, lse,
     max_logits) = _decode_prep(q, kv_cache, block_table, cache_seqlens, indices, d_v, attn_sink,
                                topk_length, out, lse, max_logits, return_max_logits)
    st = lib.sparse_mla_decode_fwd_split_noalloc(
        _p(q), _p(kv_cache), _p(block_table), _p(cache_seqlens), _p(indices), _p(topk_length),
        _p(attn_sink), B, s_q, h_q, h_kv, d_qk, d_v, topk, num_blocks, page_size,
        block_table.shape[1], float(sm_scale), int(num_splits), _p(out), _p(lse), _p(max_logits),
        _stream(dev, stream))
    _check(lib, st)
    return out, lse, max_logits


def row_lengths(indices, topk_length=None, cache_seqlens=None, *, s_kv=0, rows_per_seq=1,
                max_blocks_per_seq=0, stream=None):
    """Row lengths L as the kernels use them.  indices [..., topk] int32."""
    lib = load_library()
    dev = indices.device
    topk = indices.shape[-1]
    rows = indices.numel() // topk if topk > 0 else 0
    if topk_length is not None and topk_length.numel() != rows:
        raise ValueError("topk_length must hold one entry per row")
    if cache_seqlens is not None:
        # row r reads cache_seqlens[r // rows_per_seq]
        if rows_per_seq <= 0 or cache_seqlens.numel() * rows_per_seq < rows:
            raise ValueError(f"cache_seqlens holds {cache_seqlens.numel()} entries; {rows} rows at "
                             f"rows_per_seq={rows_per_seq} need {-(-rows // max(rows_per_seq, 1))}")
        if max_blocks_per_seq <= 0:
            raise ValueError("max_blocks_per_seq must be positive with cache_seqlens")
    _dev(indices, "indices", torch.int32)
    _dev(topk_length, "topk_length", torch.int32, dev)
    _dev(cache_seqlens, "cache_seqlens", torch.int32, dev)
    out = torch.empty(rows, dtype=torch.int32, device=dev)
    st = lib.sparse_mla_row_lengths(_p(indices), _p(topk_length), _p(cache_seqlens), rows,
                                    rows_per_seq, topk, s_kv, max_blocks_per_seq, _p(out),
                                    _stream(dev, stream))
    _check(lib, st)
    return out


def bwd_workspace_bytes(s_q, s_kv, d_qk):
    """Workspace bytes sparse_mla_bwd needs."""
    return int(load_library().sparse_mla_bwd_workspace_bytes(s_q, s_kv, d_qk))


def bwd(q, kv, out, dout, indices, lse, sm_scale, d_v=512, attn_sink=None, topk_length=None, *,
        lse_base2=False, want_d_sink=False, workspace=None, dq=None, dkv=None, stream=None):
    """Sparse prefill backward.  q [s_q, h_q, d_qk], kv [s_kv, 1, d_qk],
    out / dout [s_q, h_q, d_v] bf16; indices [s_q, 1, topk] int32; lse
    [s_q, h_q] fp32 (the forward's); attn_sink [h_q] fp32 or None.  Returns
    (dq, dkv, d_sink or None)."""
    lib = load_library()
    dev = q.device
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16, dev)
    _dev(out, "out", torch.bfloat16, dev)
    _dev(dout, "dout", torch.bfloat16, dev)
    _dev(indices, "indices", torch.int32, dev)
    _dev(lse, "lse", torch.float32, dev)
    _dev(topk_length, "topk_length", torch.int32, dev)
    _dev(attn_sink, "attn_sink", torch.float32, dev)
    if q.dim() != 3 or kv.dim() != 3 or indices.dim() != 3:
        raise ValueError("q, kv and indices must be 3-d")
    s_q, h_q, d_qk = q.shape
    s_kv, h_kv = kv.shape[0], kv.shape[1]
    topk = indices.shape[-1]
    if kv.shape[2] != d_qk or indices.shape[0] != s_q or indices.shape[1] != h_kv:
        raise ValueError("inconsistent shapes of q, kv and indices")
    if tuple(out.shape) != (s_q, h_q, d_v) or tuple(dout.shape) != (s_q, h_q, d_v):
        raise ValueError("out and dout must have shape [s_q, h_q, d_v]")
    if tuple(lse.shape) != (s_q, h_q):
        raise ValueError("lse must have shape [s_q, h_q]")
    if topk_length is not None and tuple(topk_length.shape) != (s_q,):
        raise ValueError("topk_length must have shape [s_q]")
    if attn_sink is not None and tuple(attn_sink.shape) != (h_q,):
        raise ValueError("attn_sink must have shape [h_q]")
    if want_d_sink and attn_sink is None:
        raise ValueError("d_sink needs attn_sink")
    nbytes = int(lib.sparse_mla_bwd_workspace_bytes(s_q, s_kv, d_qk))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dkv = torch.empty_like(kv) if dkv is None else dkv
    _dev(dq, "dq", torch.bfloat16, dev)
    _dev(dkv, "dkv", torch.bfloat16, dev)
    if dq.numel() != q.numel() or dkv.numel() != kv.numel():
        raise ValueError("output buffers have the wrong size")
    d_sink = torch.empty(h_q, dtype=torch.float32, device=dev) if want_d_sink else None
    st = lib.sparse_mla_bwd(_p(q), _p(kv), _p(out), _p(dout), _p(indices), _p(topk_length),
                            _p(lse), _p(attn_sink), s_q, s_kv, h_q, h_kv, d_qk, d_v, topk,
                            float(sm_scale), int(bool(lse_base2)), _p(workspace),
                            workspace.numel(), _p(dq), _p(dkv), _p(d_sink), _stream(dev, stream))
    _check(lib, st)
    return dq, dkv, d_sink


def block_sparse_fwd(q, k, v, q2k_row_ptr, q2k_col_idx, q_block, k_block, sm_scale, causal=True,
                     *, out=None, lse=None, stream=None):
    """Block-sparse forward.  q [s, h_q, 192], k [s, h_kv, 192],
    v [s, h_kv, 128] bf16; q2k_row_ptr [ceil(s / q_block) + 1] and
    q2k_col_idx [nnz] int32 (the key-block ids of each query block).
    Returns (out [s, h_q, 128] bf16, lse [s, h_q] fp32)."""
    lib = load_library()
    dev = q.device
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16, dev)
    _dev(v, "v", torch.bfloat16, dev)
    _dev(q2k_row_ptr, "q2k_row_ptr", torch.int32, dev)
    if q2k_col_idx is not None and q2k_col_idx.numel() == 0:
        q2k_col_idx = None
    _dev(q2k_col_idx, "q2k_col_idx", torch.int32, dev)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be 3-d ([s, h, d])")
    s, h_q, d_qk = q.shape
    h_kv, d_v = k.shape[1], v.shape[2]
    if k.shape[0] != s or v.shape[0] != s or k.shape[2] != d_qk or v.shape[1] != h_kv:
        raise ValueError("inconsistent shapes of q, k and v")
    if q2k_row_ptr.numel() != -(-s // q_block) + 1:
        raise ValueError("q2k_row_ptr must have ceil(s / q_block) + 1 entries")
    out = torch.empty((s, h_q, d_v), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((s, h_q), dtype=torch.float32, device=dev) if lse is None else lse
    _dev(out, "out", torch.bfloat16, dev)
    _dev(lse, "lse", torch.float32, dev)
    if out.numel() != s * h_q * d_v or lse.numel() != s * h_q:
        raise ValueError("output buffers have the wrong size")
    st = lib.sparse_mla_block_sparse_fwd(_p(q), _p(k), _p(v), _p(q2k_row_ptr), _p(q2k_col_idx), s,
                                         h_q, h_kv, d_qk, d_v, int(q_block), int(k_block),
                                         int(bool(causal)), float(sm_scale), _p(out), _p(lse),
                                         _stream(dev, stream))
    _check(lib, st)
    return out, lse


def last_kernel():
    """Name of the attention kernel the last forward, decode or backward call
    on this thread launched ("ring", "wide", "ring_split", "split", "heads16",
    all but the last with "_big" for KV tables above 4 GiB; "bwd_key_outer" or
    "bwd_scatter" for the backward's dkv path; "" for none)."""
    return load_library().sparse_mla_last_kernel().decode()
