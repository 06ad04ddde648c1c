"""Split-KV decode through the entry point that allocates nothing
(sparse_mla_decode_fwd_split_noalloc, partials in the library's static device
array) against the entry point with a caller-owned workspace
(sparse_mla_decode_fwd_split), through the C ABI, on two calls in a row, the
second with a smaller input: outputs are bitwise those of the workspace path
(same kernels, same split count) and within the parity bar of the oracle."""
import pytest
import torch

import oracle
import sparse_top_mla_amd as smla
from sparse_top_mla_amd import workloads as W
from parity import assert_bitwise, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(name, seqlens, s_q, h_q, d_qk, effective, seed):
    return W.make_decode(name, batch=len(seqlens), s_q=s_q, h_q=h_q, d_qk=d_qk, d_v=512,
                         topk=2048, seqlens=torch.tensor(seqlens), seed=seed, effective=effective,
                         with_length=True, with_sink=True)


def _run(fn, c, splits, **kw):
    q, kv, bt, cs, idx, tl, sk = (None if t is None else t.to(DEV) for t in (
        c.q, c.kv_cache, c.block_table, c.cache_seqlens, c.indices, c.topk_length, c.attn_sink))
    res = fn(q, kv, bt, cs, idx, c.sm_scale, splits, c.d_v, attn_sink=sk, topk_length=tl, **kw)
    torch.cuda.synchronize()
    return res


def _oracle(c):
    return oracle.sparse_mla_decode_fwd(c.q, c.kv_cache, c.block_table, c.cache_seqlens, c.indices,
                                        c.sm_scale, c.d_v, attn_sink=c.attn_sink,
                                        topk_length=c.topk_length)


@pytest.mark.parametrize("h_q,d_qk", [(128, 576), (64, 512)])
def test_noalloc_matches_workspace_path_on_two_calls(h_q, d_qk):
    big = _case(f"noalloc_big_h{h_q}", [2500, 4096, 1500], 2, h_q, d_qk, 1400, seed=61 + h_q)
    small = _case(f"noalloc_small_h{h_q}", [900], 2, h_q, d_qk, 700, seed=62 + h_q)
    for c, splits in ((big, 8), (small, 3)):
        print(f"[case] {c.name} splits={splits}", flush=True)
        ref = _run(smla.decode_fwd_split, c, splits)
        got = _run(smla.decode_fwd_split_noalloc, c, splits)
        assert_bitwise(ref, got, f"{c.name} no-alloc vs workspace")
        assert_parity(got, _oracle(c), c.name)


def test_noalloc_without_max_logits_and_unsplit():
    c = _case("noalloc_misc", [3000, 2100], 1, 128, 576, 1100, seed=63)
    full = _run(smla.decode_fwd_split_noalloc, c, 6)
    out, lse, ml = _run(smla.decode_fwd_split_noalloc, c, 6, return_max_logits=False)
    assert ml is None and torch.equal(out, full[0]) and torch.equal(lse, full[1])
    one = _run(smla.decode_fwd_split_noalloc, c, 1)
    assert_bitwise(one, _run(smla.decode_fwd_split, c, 1), "num_splits = 1")
    assert_parity(full, _oracle(c), c.name)
