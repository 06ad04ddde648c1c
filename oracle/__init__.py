"""CPU oracle for sparse top-k MLA attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
this package.  The product library never imports it and shares no code with
it.  The arithmetic lives in ``sparse_mla_oracle.c`` (plain C, fp64); this
module only compiles that file with gcc, loads it with ctypes and marshals
torch/numpy CPU arrays in and out.

Parity status per function (what pins it is listed in tests/oracle_pins.py):
  row_lengths          pinned (page fixtures, brute force on tiny inputs)
  sparse_mla_fwd       pinned (dense library attention, multiplicity brute
                       force, closed forms, sink closed form)
  sparse_mla_decode_fwd pinned (paged == prefill on a numpy-gathered cache,
                       dense library attention on contiguous pages)
  block_sparse_fwd     pinned (torch SDPA for full causal / full selections,
                       numpy dense-mask brute force, empty rows)
  sparse_mla_bwd       pinned (float64 autograd of dense attention with the
                       multiplicity bias, with and without a sink column;
                       single-key closed form; base-2 lse; selections)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "sparse_mla_oracle.c"
LIBRARY = _HERE / "libsparse_mla_oracle.so"

_lib = None


def build(source: Path = SOURCE, output: Path = LIBRARY, extra_flags=()) -> Path:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-shared", "-fPIC",
           *extra_flags, str(source), "-o", str(output), "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(lib):
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.oracle_row_lengths.argtypes = [vp, vp, vp, i64, i64, i32, i64, i64, vp]
    lib.oracle_row_lengths.restype = ctypes.c_int
    lib.oracle_sparse_mla_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, dbl,
                                          vp, i64, vp, vp, vp, vp, ctypes.c_int]
    lib.oracle_sparse_mla_fwd.restype = ctypes.c_int
    lib.oracle_sparse_mla_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32,
                                                 i32, i32, i64, i32, i32, dbl, vp, i64, vp, vp,
                                                 vp, vp, ctypes.c_int]
    lib.oracle_sparse_mla_decode_fwd.restype = ctypes.c_int
    lib.oracle_sparse_mla_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32,
                                          i32, dbl, ctypes.c_int, vp, i64, vp, i64, vp, vp, vp,
                                          ctypes.c_int]
    lib.oracle_sparse_mla_bwd.restype = ctypes.c_int
    lib.oracle_block_sparse_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_int, dbl, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_block_sparse_fwd.restype = ctypes.c_int
    return lib


def load(path: Path | None = None):
    """Load (building first if needed) the oracle library.  A path other than
    the default loads that library instead (used to check planted mistakes)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(str(path)))
    if _lib is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _lib = _bind(ctypes.CDLL(str(LIBRARY)))
    return _lib


def _np(x, dtype):
    """torch / numpy -> contiguous numpy of the given dtype (bf16 as raw uint16)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(threads):
    return int(threads) if threads else 0


def row_lengths(indices, topk_length=None, cache_seqlens=None, *, s_kv=0, rows_per_seq=1,
                addressable=None, lib=None):
    """Effective length of every index row.  indices: [..., topk] int32."""
    lib = lib or load()
    idx = _np(indices, np.int32)
    topk = idx.shape[-1]
    rows = idx.size // topk
    tl = _np(topk_length, np.int32)
    cs = _np(cache_seqlens, np.int32)
    if addressable is None:
        addressable = np.iinfo(np.int64).max
    out = np.empty(rows, dtype=np.int32)
    rc = lib.oracle_row_lengths(_ptr(idx), _ptr(tl), _ptr(cs), rows, rows_per_seq, topk, s_kv,
                                addressable, _ptr(out))
    if rc:
        raise ValueError(f"oracle_row_lengths failed ({rc})")
    return out


def sparse_mla_fwd(q, kv, indices, sm_scale, d_v, attn_sink=None, topk_length=None,
                   rows=None, threads=None, lib=None):
    """Prefill oracle.  q [s_q, h_q, d_qk] bf16; kv [s_kv, 1, d_qk] bf16;
    indices [s_q, 1, topk] int32.  Returns (out [n, h_q, d_v] f64,
    lse [n, h_q] f64, max_logits [n, h_q] f64, row_len [n] int32) for the
    selected rows (all rows when `rows` is None)."""
    lib = lib or load()
    qn = _np(q, np.uint16)
    kvn = _np(kv, np.uint16)
    idx = _np(indices, np.int32)
    s_q, h_q, d_qk = qn.shape
    s_kv = kvn.shape[0]
    topk = idx.shape[-1]
    sel = None if rows is None else _np(rows, np.int64)
    n = s_q if sel is None else sel.size
    out = np.empty((n, h_q, d_v), dtype=np.float64)
    lse = np.empty((n, h_q), dtype=np.float64)
    ml = np.empty((n, h_q), dtype=np.float64)
    rl = np.empty(n, dtype=np.int32)
    sink = _np(attn_sink, np.float32)
    tl = _np(topk_length, np.int32)
    rc = lib.oracle_sparse_mla_fwd(_ptr(qn), _ptr(kvn), _ptr(idx), _ptr(tl), _ptr(sink), s_q, s_kv,
                                   h_q, d_qk, d_v, topk, float(sm_scale), _ptr(sel), n, _ptr(out),
                                   _ptr(lse), _ptr(ml), _ptr(rl), _threads(threads))
    if rc:
        raise ValueError(f"oracle_sparse_mla_fwd failed ({rc})")
    return out, lse, ml, rl


def sparse_mla_decode_fwd(q, kv_cache, block_table, cache_seqlens, indices, sm_scale, d_v,
                          attn_sink=None, topk_length=None, rows=None, threads=None, lib=None):
    """Paged decode oracle.  q [B, s_q, h_q, d_qk] bf16;
    kv_cache [num_blocks, page_size, 1, d_qk] bf16; block_table [B, mbps];
    cache_seqlens [B]; indices [B, s_q, topk]; topk_length [B, s_q] or None.
    Rows are r = b * s_q + t.  Returns (out, lse, max_logits, row_len) packed
    over the selected rows."""
    lib = lib or load()
    qn = _np(q, np.uint16)
    kvn = _np(kv_cache, np.uint16)
    bt = _np(block_table, np.int32)
    cs = _np(cache_seqlens, np.int32)
    idx = _np(indices, np.int32)
    B, s_q, h_q, d_qk = qn.shape
    num_blocks, page_size = kvn.shape[0], kvn.shape[1]
    mbps = bt.shape[1]
    topk = idx.shape[-1]
    sel = None if rows is None else _np(rows, np.int64)
    n = B * s_q if sel is None else sel.size
    out = np.empty((n, h_q, d_v), dtype=np.float64)
    lse = np.empty((n, h_q), dtype=np.float64)
    ml = np.empty((n, h_q), dtype=np.float64)
    rl = np.empty(n, dtype=np.int32)
    sink = _np(attn_sink, np.float32)
    tl = _np(topk_length, np.int32)
    rc = lib.oracle_sparse_mla_decode_fwd(_ptr(qn), _ptr(kvn), _ptr(bt), _ptr(cs), _ptr(idx),
                                          _ptr(tl), _ptr(sink), B, s_q, h_q, d_qk, d_v, topk,
                                          num_blocks, page_size, mbps, float(sm_scale), _ptr(sel),
                                          n, _ptr(out), _ptr(lse), _ptr(ml), _ptr(rl),
                                          _threads(threads))
    if rc:
        raise ValueError(f"oracle_sparse_mla_decode_fwd failed ({rc})")
    return out, lse, ml, rl


def sparse_mla_bwd(q, kv, out, dout, indices, lse, sm_scale, d_v, attn_sink=None,
                   topk_length=None, lse_base2=False, rows=None, kv_rows=None, want_dq=True,
                   want_dkv=True, want_d_sink=False, threads=None, lib=None):
    """Backward oracle.  q [s_q, h_q, d_qk] bf16; kv [s_kv, 1, d_qk] bf16;
    out, dout [s_q, h_q, d_v] (bf16 or float; widened to float64);
    indices [s_q, 1, topk]; lse [s_q, h_q] (natural log, or base 2 with
    lse_base2).  Returns (dq [n, h_q, d_qk] f64 or None, dkv [n_kv, d_qk] f64
    or None, d_sink [h_q] f64 or None); `rows` / `kv_rows` select the query
    rows of dq and the KV rows of dkv (all when None)."""
    lib = lib or load()
    qn = _np(q, np.uint16)
    kvn = _np(kv, np.uint16)
    s_q, h_q, d_qk = qn.shape
    s_kv = kvn.shape[0]
    idx = _np(indices, np.int32)
    topk = idx.shape[-1]
    on = _f64_array(out).reshape(s_q, h_q, d_v)
    don = _f64_array(dout).reshape(s_q, h_q, d_v)
    ln = _f64_array(lse).reshape(s_q, h_q)
    sel = None if rows is None else _np(rows, np.int64)
    ksel = None if kv_rows is None else _np(kv_rows, np.int64)
    n = s_q if sel is None else sel.size
    nk = s_kv if ksel is None else ksel.size
    dq = np.empty((n, h_q, d_qk)) if want_dq else None
    dkv = np.empty((nk, d_qk)) if want_dkv else None
    ds = np.empty(h_q) if want_d_sink else None
    sink = _np(attn_sink, np.float32)
    tl = _np(topk_length, np.int32)
    rc = lib.oracle_sparse_mla_bwd(_ptr(qn), _ptr(kvn), _ptr(on), _ptr(don), _ptr(idx), _ptr(tl),
                                   _ptr(ln), _ptr(sink), s_q, s_kv, h_q, d_qk, d_v, topk,
                                   float(sm_scale), int(bool(lse_base2)), _ptr(sel), n,
                                   _ptr(ksel), nk, _ptr(dq), _ptr(dkv), _ptr(ds),
                                   _threads(threads))
    if rc:
        raise ValueError(f"oracle_sparse_mla_bwd failed ({rc})")
    return dq, dkv, ds


def _f64_array(x):
    """torch (any float dtype, bf16 included) / numpy -> contiguous float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def block_sparse_fwd(q, k, v, q2k_row_ptr, q2k_col_idx, q_block, k_block, sm_scale, causal=True,
                     rows=None, threads=None, lib=None):
    """Block-sparse forward oracle.  q [s, h_q, d_qk], k [s, h_kv, d_qk],
    v [s, h_kv, d_v] bf16; q2k_row_ptr [ceil(s / q_block) + 1], q2k_col_idx
    [nnz] int32.  Returns (out [n, h_q, d_v] f64, lse [n, h_q] f64) for the
    selected rows (all when None)."""
    lib = lib or load()
    qn, kn, vn = _np(q, np.uint16), _np(k, np.uint16), _np(v, np.uint16)
    s, h_q, d_qk = qn.shape
    h_kv, d_v = kn.shape[1], vn.shape[2]
    rp = _np(q2k_row_ptr, np.int32)
    ci = _np(q2k_col_idx, np.int32)
    if ci.size == 0:
        ci = np.zeros(1, dtype=np.int32)
    sel = None if rows is None else _np(rows, np.int64)
    n = s if sel is None else sel.size
    out = np.empty((n, h_q, d_v))
    lse = np.empty((n, h_q))
    rc = lib.oracle_block_sparse_fwd(_ptr(qn), _ptr(kn), _ptr(vn), _ptr(rp), _ptr(ci), s, h_q, h_kv,
                                     d_qk, d_v, int(q_block), int(k_block), int(bool(causal)),
                                     float(sm_scale), _ptr(sel), n, _ptr(out), _ptr(lse),
                                     _threads(threads))
    if rc:
        raise ValueError(f"oracle_block_sparse_fwd failed ({rc})")
    return out, lse
