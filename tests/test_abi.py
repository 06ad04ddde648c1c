"""The C-ABI library: it loads, exports every function include/sparse_mla.h
declares, and rejects bad arguments on the host before anything is launched
(CPU only: every call here returns before touching the GPU)."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "sparse_mla.h"


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_mla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_top_mla_amd import _binding, build
    if not _binding.LIBRARY.exists():
        build.build()
    return _binding.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == ["sparse_mla_block_sparse_fwd", "sparse_mla_bwd",
                                     "sparse_mla_bwd_workspace_bytes",
                                     "sparse_mla_decode_fwd", "sparse_mla_decode_fwd_split",
                                     "sparse_mla_decode_fwd_split_noalloc",
                                     "sparse_mla_decode_split_noalloc_max_bytes",
                                     "sparse_mla_decode_split_workspace_bytes", "sparse_mla_fwd",
                                     "sparse_mla_last_error", "sparse_mla_last_kernel",
                                     "sparse_mla_row_lengths"]


def test_every_declared_symbol_is_exported(lib):
    import sparse_top_mla_amd
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(sparse_top_mla_amd.EXPORTS) == set(_declared_functions())


def test_library_holds_gfx950_code_only():
    from sparse_top_mla_amd import _binding
    data = _binding.LIBRARY.read_bytes()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_90"):
        assert other not in data


NULL = None
P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first


def _fwd(lib, **kw):
    a = dict(q=P, kv=P, indices=P, topk_length=NULL, attn_sink=NULL, s_q=4, s_kv=64, h_q=64,
             h_kv=1, d_qk=576, d_v=512, topk=64, sm_scale=0.1, out=P, lse=P, max_logits=P,
             stream=NULL)
    a.update(kw)
    return lib.sparse_mla_fwd(*a.values())


def _dec(lib, **kw):
    a = dict(q=P, kv_cache=P, block_table=P, cache_seqlens=P, indices=P, topk_length=NULL,
             attn_sink=NULL, B=2, s_q=1, h_q=128, h_kv=1, d_qk=576, d_v=512, topk=64,
             num_blocks=8, page_size=64, max_blocks_per_seq=4, sm_scale=0.1, out=P, lse=P,
             max_logits=P, stream=NULL)
    a.update(kw)
    return lib.sparse_mla_decode_fwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(kv=NULL), 1), (dict(indices=NULL), 1), (dict(out=NULL), 1),
    (dict(kv=NULL, s_kv=-1), 2),
    (dict(lse=NULL), 1), (dict(max_logits=NULL), 1),
    (dict(s_q=-1), 2), (dict(s_kv=-1), 2), (dict(topk=0), 2), (dict(h_q=0), 2),
    (dict(d_v=640), 2),
    (dict(h_kv=2), 3), (dict(d_qk=128, d_v=128), 3), (dict(d_v=256), 3), (dict(h_q=24), 3),
    (dict(h_q=144), 3), (dict(sm_scale=0.0), 3), (dict(sm_scale=-0.5), 3),
    (dict(sm_scale=float("inf")), 3), (dict(sm_scale=float("nan")), 3),
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.sparse_mla_last_error().decode()


def test_fwd_empty_batch_is_noop(lib):
    assert _fwd(lib, s_q=0) == 0
    assert _fwd(lib, s_q=0, q=NULL, indices=NULL, out=NULL, lse=NULL, max_logits=NULL) == 0
    assert lib.sparse_mla_last_error().decode() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(block_table=NULL), 1), (dict(cache_seqlens=NULL), 1), (dict(kv_cache=NULL), 1),
    (dict(B=-1), 2), (dict(s_q=0), 2), (dict(max_blocks_per_seq=0), 2), (dict(num_blocks=-1), 2),
    (dict(page_size=32), 3), (dict(num_blocks=1 << 26), 3), (dict(d_qk=512, d_v=512, h_kv=3), 3),
    (dict(sm_scale=-1.0), 3),
])
def test_decode_rejects(lib, kw, status):
    assert _dec(lib, **kw) == status


def test_decode_max_logits_is_optional(lib):
    """max_logits may be NULL (the pages' decode returns out and lse only):
    the host check names out and lse as the required outputs, not it."""
    for call in (_dec, _split):
        assert call(lib, lse=NULL, max_logits=NULL) == 1
        msg = lib.sparse_mla_last_error().decode()
        assert "out and lse are required" in msg and "max_logits" not in msg


def test_decode_empty_batch_is_noop(lib):
    assert _dec(lib, B=0) == 0
    assert _dec(lib, B=0, q=NULL, indices=NULL, out=NULL, block_table=NULL) == 0


def _split(lib, **kw):
    a = dict(q=P, kv_cache=P, block_table=P, cache_seqlens=P, indices=P, topk_length=NULL,
             attn_sink=NULL, B=2, s_q=1, h_q=128, h_kv=1, d_qk=576, d_v=512, topk=64,
             num_blocks=8, page_size=64, max_blocks_per_seq=4, sm_scale=0.1, num_splits=4,
             workspace=P, workspace_bytes=1 << 30, out=P, lse=P, max_logits=P, stream=NULL)
    a.update(kw)
    return lib.sparse_mla_decode_fwd_split(*a.values())


def test_split_workspace_bytes(lib):
    f = lib.sparse_mla_decode_split_workspace_bytes
    assert f(2, 3, 128, 512, 5) == 2 * 3 * 5 * 128 * 514 * 4
    assert f(2, 3, 128, 512, 1) == 0 and f(0, 3, 128, 512, 4) == 0 and f(2, 3, 128, 512, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_splits=0), 2), (dict(num_splits=1025), 2), (dict(num_splits=-3), 2),
    (dict(workspace=NULL), 1),
    (dict(workspace_bytes=2 * 1 * 4 * 128 * 514 * 4 - 1), 2),
    (dict(workspace=ctypes.c_void_p(24)), 2),
    (dict(h_q=64), 3), (dict(h_q=96, d_qk=512), 3),
    (dict(q=NULL), 1), (dict(page_size=32), 3), (dict(B=-1), 2),
    (dict(B=1 << 20, s_q=1 << 4, num_splits=2), 2),
])
def test_split_decode_rejects(lib, kw, status):
    assert _split(lib, **kw) == status
    assert lib.sparse_mla_last_error().decode()


def test_split_decode_empty_batch_is_noop(lib):
    assert _split(lib, B=0, workspace=NULL, workspace_bytes=0) == 0


def _split_noalloc(lib, **kw):
    a = dict(q=P, kv_cache=P, block_table=P, cache_seqlens=P, indices=P, topk_length=NULL,
             attn_sink=NULL, B=2, s_q=1, h_q=128, h_kv=1, d_qk=576, d_v=512, topk=64,
             num_blocks=8, page_size=64, max_blocks_per_seq=4, sm_scale=0.1, num_splits=4,
             out=P, lse=P, max_logits=P, stream=NULL)
    a.update(kw)
    return lib.sparse_mla_decode_fwd_split_noalloc(*a.values())


def test_split_noalloc_limit(lib):
    """The static partials array holds 256 (row, split) units at 128 heads;
    larger requests are rejected on the host before any device work."""
    cap = lib.sparse_mla_decode_split_noalloc_max_bytes()
    assert cap == 256 * 128 * 514 * 4
    assert lib.sparse_mla_decode_split_workspace_bytes(64, 1, 128, 512, 4) <= cap
    assert _split_noalloc(lib, B=65, num_splits=4) == 2
    assert "static scratch array" in lib.sparse_mla_last_error().decode()
    assert _split_noalloc(lib, B=2, s_q=2, num_splits=65) == 2


@pytest.mark.parametrize("kw,status", [
    (dict(num_splits=0), 2), (dict(num_splits=1025), 2), (dict(q=NULL), 1), (dict(lse=NULL), 1),
    (dict(page_size=32), 3), (dict(B=-1), 2),
])
def test_split_noalloc_rejects(lib, kw, status):
    assert _split_noalloc(lib, **kw) == status
    assert lib.sparse_mla_last_error().decode()


def test_split_noalloc_empty_batch_is_noop(lib):
    assert _split_noalloc(lib, B=0, out=NULL, lse=NULL, max_logits=NULL) == 0


def _bwd(lib, **kw):
    a = dict(q=P, kv=P, out=P, dout=P, indices=P, topk_length=NULL, lse=P, attn_sink=NULL,
             s_q=8, s_kv=64, h_q=64, h_kv=1, d_qk=576, d_v=512, topk=32, sm_scale=0.1,
             lse_base2=0, workspace=P, workspace_bytes=1 << 30, dq=P, dkv=P, d_sink=NULL,
             stream=NULL)
    a.update(kw)
    return lib.sparse_mla_bwd(*a.values())


def test_bwd_workspace_bytes(lib):
    f = lib.sparse_mla_bwd_workspace_bytes
    # fp32 accumulator and row lengths, then (s_kv <= 16384, s_q * s_kv <=
    # 2^28) the key-outer buffers: statistics [s_q][128] fp32, flags [s_q],
    # bitmaps [s_q][ceil(s_kv / 32)] words; each part rounded up to 256 bytes.
    assert f(8, 64, 576) == 64 * 576 * 4 + 256 + 8 * 128 * 4 + 256 + 256
    assert f(300, 1, 512) == 2048 + 1280 + 300 * 128 * 4 + 1280 + 1280
    assert f(8, 20000, 576) == 20000 * 576 * 4 + 256
    assert f(0, 0, 576) == 0 and f(-1, 4, 576) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=32), 3), (dict(h_q=128), 3), (dict(d_qk=320), 3), (dict(d_v=256), 3),
    (dict(h_kv=2), 3), (dict(sm_scale=0.0), 3), (dict(sm_scale=float("nan")), 3),
    (dict(topk=0), 2), (dict(s_q=-1), 2), (dict(s_kv=-5), 2), (dict(lse_base2=2), 2),
    (dict(d_sink=P), 1), (dict(workspace=NULL), 1),
    (dict(workspace_bytes=64 * 576 * 4 + 255), 2), (dict(workspace=ctypes.c_void_p(24)), 2),
    (dict(q=NULL), 1), (dict(lse=NULL), 1), (dict(dkv=NULL), 1), (dict(dq=NULL), 1),
])
def test_bwd_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status
    assert lib.sparse_mla_last_error().decode()


def test_bwd_empty_is_noop(lib):
    assert _bwd(lib, s_q=0, s_kv=0, workspace=NULL, workspace_bytes=0) == 0


def _bs(lib, **kw):
    a = dict(q=P, k=P, v=P, row_ptr=P, col_idx=P, s=512, h_q=8, h_kv=8, d_qk=192, d_v=128,
             q_block=256, k_block=128, causal=1, sm_scale=0.07, out=P, lse=P, stream=NULL)
    a.update(kw)
    return lib.sparse_mla_block_sparse_fwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(d_qk=576), 3), (dict(d_v=512), 3), (dict(q_block=100), 3), (dict(k_block=32), 3),
    (dict(q_block=0), 3), (dict(h_kv=3), 2), (dict(h_q=0), 2), (dict(s=-1), 2),
    (dict(causal=2), 2), (dict(sm_scale=-1.0), 3), (dict(q=NULL), 1), (dict(row_ptr=NULL), 1),
    (dict(lse=NULL), 1),
])
def test_block_sparse_rejects(lib, kw, status):
    assert _bs(lib, **kw) == status
    assert lib.sparse_mla_last_error().decode()


def test_block_sparse_empty_is_noop(lib):
    assert _bs(lib, s=0, q=NULL, k=NULL, v=NULL, row_ptr=NULL, out=NULL, lse=NULL) == 0


def test_row_lengths_rejects(lib):
    f = lib.sparse_mla_row_lengths
    assert f(NULL, NULL, NULL, 4, 1, 64, 10, 0, P, NULL) == 1
    assert f(P, NULL, NULL, 4, 1, 0, 10, 0, P, NULL) == 2
    assert f(P, NULL, P, 4, 1, 64, 10, 0, P, NULL) == 2
    assert f(P, NULL, NULL, 0, 1, 64, 10, 0, P, NULL) == 0


def test_binding_row_lengths_checks_seqlens():
    """row r reads cache_seqlens[r // rows_per_seq]: the binding rejects a
    cache_seqlens tensor too short for the rows, before anything runs."""
    import torch
    import sparse_top_mla_amd as smla
    idx = torch.zeros(4, 2, 64, dtype=torch.int32)   # 8 rows
    with pytest.raises(ValueError, match="cache_seqlens"):
        smla.row_lengths(idx, cache_seqlens=torch.zeros(4, dtype=torch.int32), max_blocks_per_seq=4)
    with pytest.raises(ValueError, match="cache_seqlens"):
        smla.row_lengths(idx, cache_seqlens=torch.zeros(3, dtype=torch.int32), rows_per_seq=2,
                         max_blocks_per_seq=4)
    with pytest.raises(ValueError, match="max_blocks_per_seq"):
        smla.row_lengths(idx, cache_seqlens=torch.zeros(4, dtype=torch.int32), rows_per_seq=2)
    with pytest.raises(ValueError, match="topk_length"):
        smla.row_lengths(idx, topk_length=torch.zeros(4, dtype=torch.int32))


def test_binding_rejects_cpu_tensors():
    import torch
    import sparse_top_mla_amd as smla
    q = torch.zeros(2, 16, 576, dtype=torch.bfloat16)
    kv = torch.zeros(8, 1, 576, dtype=torch.bfloat16)
    idx = torch.zeros(2, 1, 64, dtype=torch.int32)
    with pytest.raises(TypeError):
        smla.fwd(q, kv, idx, 0.1)


def test_last_kernel_is_empty_after_a_rejected_call(lib):
    from sparse_top_mla_amd import _binding
    assert _fwd(lib, s_q=-1) != 0
    assert _binding.last_kernel() == ""
