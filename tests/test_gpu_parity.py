"""HIP path vs the fp64 CPU oracle, through the C ABI (GPU only).

Tolerances are those of tests/parity.py (out max-abs 2e-2 and relative L2
1e-2; lse and max_logits 1e-3 absolute; empty rows exact; row lengths
bit-exact).  Bitwise GPU-vs-GPU checks cover the statements of the pages:
derived == explicit length (FlashMLA PR #196, "Numbers"), INT_MAX-poisoned
dynamic == -1-padded fixed (PR #216, "Dynamic top-k"), any invalid encoding
masks alike, and NaN behind an unused index never leaks.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_amd as smla
from sparse_top_mla_amd import workloads as W
from parity import assert_bitwise, assert_parity, sample_rows

pytestmark = pytest.mark.gpu

INT32_MAX = 2**31 - 1
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _to(case_tensors):
    return [None if t is None else t.to(DEV) for t in case_tensors]


def run_prefill(c, topk_length="case", sink="case"):
    tl = c.topk_length if topk_length == "case" else topk_length
    sk = c.attn_sink if sink == "case" else sink
    q, kv, idx, tl_d, sk_d = _to([c.q, c.kv, c.indices, tl, sk])
    res = smla.fwd(q, kv, idx, c.sm_scale, c.d_v, attn_sink=sk_d, topk_length=tl_d)
    torch.cuda.synchronize()
    return res


def run_decode(c, topk_length="case", indices=None, kv_cache=None):
    tl = c.topk_length if topk_length == "case" else topk_length
    idx = c.indices if indices is None else indices
    kvc = c.kv_cache if kv_cache is None else kv_cache
    q, kv, bt, cs, idx_d, tl_d, sk = _to([c.q, kvc, c.block_table, c.cache_seqlens, idx, tl,
                                          c.attn_sink])
    res = smla.decode_fwd(q, kv, bt, cs, idx_d, c.sm_scale, c.d_v, attn_sink=sk, topk_length=tl_d)
    torch.cuda.synchronize()
    return res


def oracle_prefill(c, rows=None, topk_length="case"):
    tl = c.topk_length if topk_length == "case" else topk_length
    return oracle.sparse_mla_fwd(c.q, c.kv, c.indices, c.sm_scale, c.d_v, attn_sink=c.attn_sink,
                                 topk_length=tl, rows=rows)


def oracle_decode(c, rows=None, topk_length="case"):
    tl = c.topk_length if topk_length == "case" else topk_length
    return oracle.sparse_mla_decode_fwd(c.q, c.kv_cache, c.block_table, c.cache_seqlens, c.indices,
                                        c.sm_scale, c.d_v, attn_sink=c.attn_sink, topk_length=tl,
                                        rows=rows)


# ---------------------------------------------------------------------------
# small cases: every row checked
# ---------------------------------------------------------------------------

def test_tiny_prefill():
    c = W.tiny_prefill()
    _say(c.name)
    assert_parity(run_prefill(c), oracle_prefill(c), c.name)


@pytest.mark.parametrize("with_length", [False, True])
def test_prefill_h64_ramp_window(with_length):
    # rows 996..1043 and 0..23 of the 1027-capped causal ramp, width 1152
    for off, n in ((996, 48), (0, 24)):
        c = W.prefill_h64(with_length=with_length, s_q=n, s_kv=8192, row_offset=off)
        _say(f"{c.name} rows {off}..{off + n - 1}")
        assert_parity(run_prefill(c), oracle_prefill(c), c.name)


def test_prefill_h128_scattered_sink():
    c = W.make_prefill("h128_scatter_small", s_q=24, s_kv=4096, h_q=128, d_qk=576, d_v=512,
                       topk=2048, layout="scattered", invalid_frac=0.1, empty_frac=0.125,
                       with_sink=True, seed=3)
    _say(c.name)
    assert len(c.meta["empty_rows"]) == 3
    assert_parity(run_prefill(c), oracle_prefill(c), c.name)


@pytest.mark.parametrize("h_q", [16, 32, 48, 64, 80, 96, 112, 128])
@pytest.mark.parametrize("d_qk", [512, 576])
def test_prefill_head_counts(h_q, d_qk):
    c = W.make_prefill(f"heads{h_q}_d{d_qk}", s_q=9, s_kv=300, h_q=h_q, d_qk=d_qk, d_v=512,
                       topk=200, layout="scattered", invalid_frac=0.3, empty_frac=0.12,
                       with_sink=(h_q % 32 == 0), seed=h_q + d_qk)
    _say(c.name)
    assert_parity(run_prefill(c), oracle_prefill(c), c.name)


@pytest.mark.parametrize("topk", [1, 7, 63, 64, 65, 100, 129, 300])
def test_prefill_ragged_topk(topk):
    c = W.make_prefill(f"topk{topk}", s_q=11, s_kv=5000, h_q=64, d_qk=576, d_v=512, topk=topk,
                       layout="scattered", invalid_frac=0.25, seed=topk)
    _say(c.name)
    assert_parity(run_prefill(c), oracle_prefill(c), c.name)
    lens = torch.tensor(oracle.row_lengths(c.indices, s_kv=c.s_kv), dtype=torch.int32)
    got = run_prefill(c, topk_length=lens)
    assert_bitwise(run_prefill(c), got, f"{c.name} derived vs explicit")


def _tail_rows(topk=192, s_kv=1000, seed=0, lens=None):
    """Rows whose last valid entry sits at each boundary length of FlashMLA
    PR #216, "Correctness" (0, 1, 17, 63, 64, 65, 127, 128) and a few more,
    with -1 interior holes."""
    gen = torch.Generator().manual_seed(seed)
    if lens is None:
        lens = [0, 1, 17, 63, 64, 65, 127, 128, 129, 191, 192]
    idx = torch.full((len(lens), topk), -1, dtype=torch.int64)
    for r, n in enumerate(lens):
        if n:
            idx[r, :n] = torch.randint(0, s_kv, (n,), generator=gen)
            holes = torch.rand(n, generator=gen) < 0.2
            holes[n - 1] = False
            idx[r, :n][holes] = -1
    return lens, idx.to(torch.int32)


@pytest.mark.parametrize("d_qk", [512, 576])
def test_tail_lengths_and_bitwise_equivalences(d_qk):
    lens, idx = _tail_rows()
    n = len(lens)
    c = W.make_prefill("tails", s_q=n, s_kv=1000, h_q=64, d_qk=d_qk, d_v=512, topk=192,
                       layout="full", seed=9, with_sink=True)
    c.indices = idx.view(n, 1, 192).contiguous()
    c.topk_length = None
    _say(f"tail lengths d{d_qk}")
    base = run_prefill(c)
    assert_parity(base, oracle_prefill(c), "tails derived")
    # the kernel's row lengths are the oracle's, bit for bit
    rl = smla.row_lengths(c.indices.to(DEV), s_kv=1000).cpu()
    assert rl.tolist() == lens
    assert rl.tolist() == oracle.row_lengths(c.indices, s_kv=1000).tolist()
    # derived == explicit (bitwise)
    explicit = torch.tensor(lens, dtype=torch.int32)
    assert_bitwise(base, run_prefill(c, topk_length=explicit), "derived vs explicit")
    # -1 padding without a length == INT_MAX poisoning with a length (bitwise)
    poisoned = idx.clone()
    for r, L in enumerate(lens):
        poisoned[r, L:] = INT32_MAX
    c2 = W.PrefillCase("tails_dyn", c.q, c.kv, poisoned.view(n, 1, 192).contiguous(), explicit,
                       c.attn_sink, c.sm_scale, c.d_v)
    assert_bitwise(base, run_prefill(c2), "fixed vs dynamic")
    # any invalid encoding at the same positions (bitwise)
    for enc in (-2, -(2**31), 1000, 1001, INT32_MAX):
        alt = torch.where(idx < 0, torch.full_like(idx, enc), idx)
        c3 = W.PrefillCase("enc", c.q, c.kv, alt.view(n, 1, 192).contiguous(), None, c.attn_sink,
                           c.sm_scale, c.d_v)
        assert_bitwise(base, run_prefill(c3), f"encoding {enc}")


@pytest.mark.parametrize("d_qk,with_sink", [(512, False), (512, True), (576, True)])
def test_tail_lengths_at_32_key_blocks(d_qk, with_sink):
    """The 64-head kernel at d_qk = 512 works on 32-key blocks: lengths at
    and around their edges, derived and explicit, against the oracle."""
    lens, idx = _tail_rows(seed=3, lens=[31, 32, 33, 95, 96, 97, 159, 160, 161, 2])
    n = len(lens)
    c = W.make_prefill("tails32", s_q=n, s_kv=1000, h_q=64, d_qk=d_qk, d_v=512, topk=192,
                       layout="full", seed=11, with_sink=with_sink)
    c.indices = idx.view(n, 1, 192).contiguous()
    c.topk_length = None
    _say(f"32-key tails d{d_qk} sink={with_sink}")
    base = run_prefill(c)
    assert_parity(base, oracle_prefill(c), "tails32 derived")
    explicit = torch.tensor(lens, dtype=torch.int32)
    assert_bitwise(base, run_prefill(c, topk_length=explicit), "tails32 derived vs explicit")


def test_nan_behind_unused_indices_never_leaks():
    c = W.make_prefill("nan_guard", s_q=16, s_kv=2048, h_q=64, d_qk=576, d_v=512, topk=256,
                       layout="scattered", invalid_frac=0.3, empty_frac=0.0, seed=17)
    idx = c.indices.view(16, 256).clone()
    used = torch.zeros(2048, dtype=torch.bool)
    lens = torch.full((16,), 200, dtype=torch.int32)
    for r in range(16):
        row = idx[r, :200]
        used[row[(row >= 0) & (row < 2048)].long()] = True
    _say("nan guard")
    base = run_prefill(c, topk_length=lens)
    poisoned = c.kv.clone()
    poisoned[~used] = float("nan")
    c2 = W.PrefillCase("nan", c.q, poisoned, c.indices, lens, None, c.sm_scale, c.d_v)
    got = run_prefill(c2, topk_length=lens)
    assert_bitwise(base, got, "NaN in unused rows")
    assert torch.isfinite(got[0].float()).all()


def test_prefill_no_kv_rows():
    c = W.make_prefill("s_kv0", s_q=5, s_kv=64, h_q=16, d_qk=576, d_v=512, topk=64,
                       layout="full", seed=2)
    kv0 = c.kv[:0]
    out, lse, ml = smla.fwd(c.q.to(DEV), kv0.to(DEV).contiguous(), c.indices.to(DEV), c.sm_scale)
    torch.cuda.synchronize()
    assert (out == 0).all() and (lse == math.inf).all() and (ml == -math.inf).all()


def test_empty_batch():
    q = torch.zeros(0, 64, 512, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(10, 1, 512, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(0, 1, 64, dtype=torch.int32, device=DEV)
    out, lse, ml = smla.fwd(q, kv, idx, 0.1)
    assert out.shape == (0, 64, 512)


def test_decode_dynamic_small():
    c = W.decode_dynamic(with_length=True, batch=8)
    _say(c.name)
    dyn = run_decode(c)
    assert_parity(dyn, oracle_decode(c), c.name)
    fixed = W.decode_dynamic(with_length=False, batch=8)
    assert_bitwise(dyn, run_decode(fixed), "decode fixed vs dynamic")
    # [B]-shaped lengths broadcast over s_q
    assert_bitwise(dyn, run_decode(c, topk_length=c.topk_length[:, 0].contiguous()), "[B] length")


def test_decode_fixed_small():
    c = W.decode_fixed(batch=4)
    _say(c.name)
    assert_parity(run_decode(c), oracle_decode(c), c.name)


def test_decode_edge_tables():
    """Cache lengths past the table's reach, bad page entries, short caches,
    a sink and explicit lengths, against the oracle's reading of each."""
    c = W.make_decode("decode_edges", batch=5, s_q=3, h_q=64, d_qk=576, d_v=512, topk=160,
                      seqlens=torch.tensor([700, 64, 1, 333, 129]), seed=4, effective=1,
                      with_sink=True, spare_pages=16)
    # indices: mix of valid, invalid and out-of-range
    gen = torch.Generator().manual_seed(11)
    c.indices = torch.randint(-3, 800, c.indices.shape, generator=gen).to(torch.int32)
    bt = c.block_table.clone()
    bt[0, 3] = -1                      # a hole in the table
    bt[3, 2] = c.kv_cache.shape[0]     # an entry past the pool
    c.block_table = bt
    cs = c.cache_seqlens.clone()
    cs[4] = 100000                     # beyond max_blocks_per_seq * 64
    c.cache_seqlens = cs
    # request 4 now reaches past its old length: make its last page finite
    kvc = c.kv_cache.clone()
    kvc[int(bt[4, 2])] = torch.randn(kvc.shape[1:], generator=gen).to(torch.bfloat16)
    c.kv_cache = kvc
    _say(c.name)
    assert_parity(run_decode(c), oracle_decode(c), c.name)
    tl = torch.randint(-5, 200, (5, 3), generator=gen).to(torch.int32)
    assert_parity(run_decode(c, topk_length=tl), oracle_decode(c, topk_length=tl), c.name + " len")
    rl = smla.row_lengths(c.indices.to(DEV), None, c.cache_seqlens.to(DEV), rows_per_seq=3,
                          max_blocks_per_seq=c.block_table.shape[1]).cpu().numpy()
    ref = oracle.row_lengths(c.indices, None, c.cache_seqlens, rows_per_seq=3,
                             addressable=c.block_table.shape[1] * 64)
    assert np.array_equal(rl, ref)


@pytest.mark.parametrize("h_q,num_splits", [(128, 1), (64, 1), (48, 1), (128, 4)])
def test_decode_without_max_logits(h_q, num_splits):
    """max_logits = NULL (the pages' decode returns out and lse only): out
    and lse are bitwise those of the call that stores max_logits, in the
    wide kernel (128 and 64 heads), the 16-head kernel (48) and split
    decode."""
    gen = torch.Generator().manual_seed(h_q + num_splits)
    seqlens = torch.randint(200, 700, (6,), generator=gen)
    c = W.make_decode(f"decode_no_ml_h{h_q}_s{num_splits}", batch=6, s_q=2, h_q=h_q, d_qk=576,
                      d_v=512, topk=256, seqlens=seqlens, seed=50 + h_q, effective=200,
                      with_length=True, with_sink=True)
    _say(c.name)
    q, kv, bt, cs, idx, tl, sk = _to([c.q, c.kv_cache, c.block_table, c.cache_seqlens, c.indices,
                                      c.topk_length, c.attn_sink])
    if num_splits == 1:
        full = smla.decode_fwd(q, kv, bt, cs, idx, c.sm_scale, c.d_v, attn_sink=sk, topk_length=tl)
        out, lse, ml = smla.decode_fwd(q, kv, bt, cs, idx, c.sm_scale, c.d_v, attn_sink=sk,
                                       topk_length=tl, return_max_logits=False)
    else:
        full = smla.decode_fwd_split(q, kv, bt, cs, idx, c.sm_scale, num_splits, c.d_v,
                                     attn_sink=sk, topk_length=tl)
        out, lse, ml = smla.decode_fwd_split(q, kv, bt, cs, idx, c.sm_scale, num_splits, c.d_v,
                                             attn_sink=sk, topk_length=tl,
                                             return_max_logits=False)
    torch.cuda.synchronize()
    assert ml is None
    assert torch.equal(out, full[0]) and torch.equal(lse, full[1]), c.name
    assert_parity(full, oracle_decode(c), c.name)


def test_decode_nan_pages_never_leak():
    c = W.decode_fixed(batch=3, min_len=2100, max_len=5000)
    _say("decode NaN guard")
    base = run_decode(c)
    # spare pages and tails are already NaN; additionally poison every token
    # that no row names
    kvc = c.kv_cache.clone().view(-1, 576)
    used = torch.zeros(kvc.shape[0], dtype=torch.bool)
    for b in range(c.batch):
        pos = c.indices[b].reshape(-1).long()
        pos = pos[(pos >= 0) & (pos < int(c.cache_seqlens[b]))]
        phys = c.block_table[b].long()[pos // 64] * 64 + pos % 64
        used[phys] = True
    kvc[~used] = float("nan")
    got = run_decode(c, kv_cache=kvc.view_as(c.kv_cache))
    assert_bitwise(base, got, "decode NaN poisoning")


def test_row_lengths_fixtures_on_gpu():
    from oracle_pins import _golden_rows
    for name, row, s_kv, explicit, exp_len, _ in _golden_rows():
        idx = torch.from_numpy(row).view(1, -1).to(DEV)
        tl = None if explicit is None else torch.tensor([explicit], dtype=torch.int32, device=DEV)
        got = int(smla.row_lengths(idx, tl, s_kv=s_kv).item())
        assert got == exp_len, name


def test_row_lengths_random_bitexact():
    gen = torch.Generator().manual_seed(1)
    for topk in (1, 5, 64, 255, 256, 257, 700, 2048):
        idx = torch.randint(-2, 60, (300, topk), generator=gen).to(torch.int32)
        idx[::3, topk // 2:] = -1
        idx[1::5, :] = INT32_MAX
        got = smla.row_lengths(idx.to(DEV), s_kv=50).cpu().numpy()
        assert np.array_equal(got, oracle.row_lengths(idx, s_kv=50)), topk


# ---------------------------------------------------------------------------
# more rows than the grid has workgroups (one per CU, 256 on MI355X): each
# workgroup walks several rows and prepares a row's successor under it (for
# 64 heads the successor's query slice is gathered into the last block's
# buffer).  Empty rows and both block-count parities sit between them.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("h_q,d_qk", [(64, 512), (64, 576), (128, 512), (128, 576)])
def test_prefill_rows_beyond_grid(h_q, d_qk):
    c = W.make_prefill(f"rows300_h{h_q}_d{d_qk}", s_q=300, s_kv=700, h_q=h_q, d_qk=d_qk, d_v=512,
                       topk=96, layout="scattered", invalid_frac=0.3, empty_frac=0.05,
                       with_sink=(d_qk == 576), seed=7 + h_q + d_qk)
    _say(c.name)
    assert_parity(run_prefill(c), oracle_prefill(c), c.name)
    # explicit lengths 0..96: rows of 0, 1 and 2 blocks in every order
    gen = torch.Generator().manual_seed(h_q + d_qk)
    tl = torch.randint(0, 97, (c.s_q,), generator=gen, dtype=torch.int32)
    assert_parity(run_prefill(c, topk_length=tl), oracle_prefill(c, topk_length=tl),
                  c.name + " explicit lengths")


@pytest.mark.parametrize("h_q,d_qk", [(64, 512), (64, 576), (128, 576)])
def test_persistent_grid_is_schedule_invariant(h_q, d_qk):
    """A row's result does not depend on the workgroup or the turn that
    computes it: slices of a case (other grid sizes, other snake positions)
    give the rows of the whole case bit for bit."""
    c = W.make_prefill(f"sched_h{h_q}_d{d_qk}", s_q=600, s_kv=900, h_q=h_q, d_qk=d_qk, d_v=512,
                       topk=160, layout="scattered", invalid_frac=0.2, empty_frac=0.03,
                       with_sink=True, seed=23 + h_q + d_qk)
    _say(c.name)
    whole = run_prefill(c)
    for lo, hi in ((0, 600), (37, 301), (250, 251), (599, 600), (100, 460)):
        part = W.PrefillCase(c.name, c.q[lo:hi].contiguous(), c.kv, c.indices[lo:hi].contiguous(),
                             None, c.attn_sink, c.sm_scale, c.d_v)
        got = run_prefill(part)
        ref = tuple(t[lo:hi] for t in whole)
        assert_bitwise(ref, got, f"rows {lo}..{hi - 1}")


@pytest.mark.parametrize("h_q", [64, 128])
def test_decode_rows_beyond_grid(h_q):
    gen = torch.Generator().manual_seed(h_q)
    seqlens = torch.randint(100, 900, (150,), generator=gen)
    c = W.make_decode(f"decode_rows300_h{h_q}", batch=150, s_q=2, h_q=h_q, d_qk=576, d_v=512,
                      topk=128, seqlens=seqlens, seed=h_q, effective=100, with_length=True,
                      with_sink=True)
    _say(c.name)
    dyn = run_decode(c)
    assert_parity(dyn, oracle_decode(c), c.name)
    assert_bitwise(dyn, run_decode(c, topk_length=None), f"{c.name} dynamic vs fixed")


# ---------------------------------------------------------------------------
# split-KV decode: every row's index blocks split several ways and merged
# (lse = logsumexp of the splits, the sink once after the merge)
# ---------------------------------------------------------------------------

def run_decode_split(c, num_splits, topk_length="case", workspace=None):
    tl = c.topk_length if topk_length == "case" else topk_length
    q, kv, bt, cs, idx_d, tl_d, sk = _to([c.q, c.kv_cache, c.block_table, c.cache_seqlens,
                                          c.indices, tl, c.attn_sink])
    res = smla.decode_fwd_split(q, kv, bt, cs, idx_d, c.sm_scale, num_splits, c.d_v,
                                attn_sink=sk, topk_length=tl_d, workspace=workspace)
    torch.cuda.synchronize()
    return res


def _small_batch_decode(h_q=128, d_qk=576, with_sink=True, with_length=True, seed=31):
    """The pages' small-batch decode shape (s_q = 2, topk 2048, variable KV
    lengths), at cache lengths the oracle takes in seconds."""
    seqlens = torch.tensor([2500, 4096])
    return W.make_decode(f"split_b2_h{h_q}_d{d_qk}", batch=2, s_q=2, h_q=h_q, d_qk=d_qk, d_v=512,
                         topk=2048, seqlens=seqlens, seed=seed, effective=2000,
                         with_length=with_length, with_sink=with_sink)


@pytest.mark.parametrize("num_splits", [2, 3, 7, 32, 40])
def test_split_decode_matches_oracle(num_splits):
    c = _small_batch_decode()
    _say(f"{c.name} splits={num_splits}")
    ref = oracle_decode(c)
    got = run_decode_split(c, num_splits)
    assert_parity(got, ref, f"{c.name} x{num_splits}")
    # derived lengths (INT_MAX-poisoned tails) give the same split results
    assert_bitwise(got, run_decode_split(c, num_splits, topk_length=None),
                   f"{c.name} x{num_splits} dynamic vs fixed")
    # and the unsplit path agrees within the parity tolerance
    assert_parity(run_decode(c), ref, f"{c.name} unsplit")


@pytest.mark.parametrize("h_q,d_qk,with_sink", [(128, 512, False), (64, 512, True),
                                                 (128, 576, False)])
def test_split_decode_layouts(h_q, d_qk, with_sink):
    c = _small_batch_decode(h_q=h_q, d_qk=d_qk, with_sink=with_sink, with_length=False,
                            seed=h_q + d_qk)
    _say(f"{c.name} sink={with_sink}")
    assert_parity(run_decode_split(c, 5), oracle_decode(c), c.name)


def test_split_decode_short_and_empty_rows():
    """Rows of length 0 and 1 (splits without keys), and a caller's workspace
    used twice."""
    c = _small_batch_decode(seed=5)
    tl = torch.tensor([[0, 1], [64, 2000]], dtype=torch.int32)
    _say("split decode short rows")
    ref = oracle_decode(c, topk_length=tl)
    need = smla.decode_split_workspace_bytes(2, 2, 128, 512, 9)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    a = run_decode_split(c, 9, topk_length=tl, workspace=ws)
    assert_parity(a, ref, "split short rows")
    assert_bitwise(a, run_decode_split(c, 9, topk_length=tl, workspace=ws), "workspace reused")


def test_split_decode_wide_units_at_128_heads():
    """128 heads with more than 2048 positions per split run the wide
    kernel's split units; the ring's split units take the rest."""
    seqlens = torch.tensor([5000, 4500])
    c = W.make_decode("split_wide_h128", batch=2, s_q=2, h_q=128, d_qk=576, d_v=512, topk=4160,
                      seqlens=seqlens, seed=77, effective=4100, with_length=True, with_sink=True)
    _say(c.name)
    ref = oracle_decode(c)
    got = run_decode_split(c, 2)
    assert smla.last_kernel() == "split"
    assert_parity(got, ref, c.name + " x2")
    got = run_decode_split(c, 3)
    assert smla.last_kernel() == "ring_split"
    assert_parity(got, ref, c.name + " x3")


def test_split_decode_unsupported_layout_raises():
    c = _small_batch_decode(h_q=64, d_qk=576)
    with pytest.raises(smla.SparseMLAError):
        run_decode_split(c, 4)


# ---------------------------------------------------------------------------
# the recompute: a logit far above the first tile's maximum (more than 2^64
# in exp2 units) makes the workgroup redo the row with the true maximum as
# the reference.  Head 0's query of a planted row is scaled by 10 and one key
# (after the first tile) is that row's original query, so its logit leads by
# about 290 in log2 units while V keeps ordinary magnitudes.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("h_q,d_qk", [(64, 512), (64, 576), (128, 576)])
def test_recompute_on_dominant_logit(h_q, d_qk):
    c = W.make_prefill(f"recompute_h{h_q}_d{d_qk}", s_q=300, s_kv=1200, h_q=h_q, d_qk=d_qk,
                       d_v=512, topk=192, layout="scattered", seed=41 + h_q + d_qk,
                       with_sink=True)
    idx = c.indices.view(c.s_q, c.topk)
    rows = [0, 7, 150, 263, 299]
    for j, r in enumerate(rows):
        kvr = 1100 + j                    # KV rows no other index names
        idx[r][idx[r] == kvr] = 0
        c.kv[kvr, 0] = c.q[r, 0]
        c.q[r, 0] = (10.0 * c.q[r, 0].float()).to(torch.bfloat16)
        idx[r, 100 + j] = kvr             # after the first tile (and block)
    _say(c.name)
    res = run_prefill(c)
    ref = oracle_prefill(c)
    assert np.all(ref[1][rows, 0] > ref[1][rows, 1] + 150)  # the planted logit dominates head 0
    assert_parity(res, ref, c.name)


def test_recompute_in_split_decode():
    c = _small_batch_decode(seed=43, with_length=False)
    idx = c.indices.view(4, c.topk)
    pos = 1500                            # late in the row: a later split
    for r in range(4):
        b = r // 2
        tok = int(idx[r, pos].item())
        page = int(c.block_table[b, tok // 64].item())
        c.kv_cache[page, tok % 64, 0] = c.q[b, r % 2, 0]
        c.q[b, r % 2, 0] = (10.0 * c.q[b, r % 2, 0].float()).to(torch.bfloat16)
    _say("split decode recompute")
    ref = oracle_decode(c)
    assert_parity(run_decode_split(c, 8), ref, "split recompute")
    assert_parity(run_decode(c), ref, "unsplit recompute")


# ---------------------------------------------------------------------------
# KV tables past 4 GiB (beyond 32-bit buffer offsets: the ring, wide and split
# kernels then rebase a resource per copied row): the rows of a small case are
# placed at rows or pages of a larger table, many of them past the 4 GiB mark,
# and the results must be the small case's
# ---------------------------------------------------------------------------

BIG_ROWS = (1 << 32) // 1152 + 40_000  # ~4.35 GB at d_qk = 576


# (h_q, d_qk, s_q, topk): one row per workgroup, and rows beyond the
# persistent grid (each workgroup walks two or three rows: the 64-head
# d_qk = 576 layout then loads the next row's query slice into registers);
# 128 heads with rows longer than the ring kernel takes run the wide kernel
@pytest.mark.parametrize("h_q,d_qk,s_q,topk", [(64, 576, 6, 128), (128, 576, 6, 128),
                                               (64, 576, 300, 128), (64, 512, 600, 128),
                                               (128, 512, 300, 128), (128, 576, 6, 2112)])
def test_kv_table_past_4gib(h_q, d_qk, s_q, topk):
    small = W.make_prefill(f"big_kv_h{h_q}_d{d_qk}_s{s_q}_k{topk}", s_q=s_q, s_kv=max(768, topk + 64),
                           h_q=h_q, d_qk=d_qk, d_v=512, topk=topk, layout="scattered",
                           invalid_frac=0.2, seed=5 + h_q + s_q, with_sink=True)
    rows = (1 << 32) // (2 * d_qk) + 40_000
    gen = torch.Generator().manual_seed(6)
    pos = torch.randperm(rows - 700_000, generator=gen)[:small.s_kv]
    pos[::2] = rows - 1 - torch.arange(0, small.s_kv, 2)  # half of them in the last rows
    idx = small.indices.long()
    ok = (idx >= 0) & (idx < small.s_kv)
    # invalid entries stay invalid in the big table (-1; an out-of-range value
    # of the small table may be a row of the big one)
    big_idx = torch.where(ok, pos[idx.clamp(0, small.s_kv - 1)], -1).to(torch.int32)
    kv_big = torch.zeros((rows, 1, d_qk), dtype=torch.bfloat16, device=DEV)
    kv_big[pos.to(DEV)] = small.kv.to(DEV)
    _say(small.name)
    sk = small.attn_sink.to(DEV)
    res = smla.fwd(small.q.to(DEV), kv_big, big_idx.to(DEV), small.sm_scale, small.d_v,
                   attn_sink=sk)
    ring = h_q == 128 and topk <= 2048
    assert smla.last_kernel() == ("ring_big" if ring else "wide_big")
    torch.cuda.synchronize()
    assert_parity(res, oracle_prefill(small), small.name + " in a >4 GiB table")
    # the same case in its own small table takes the 32-bit form
    smla.fwd(small.q.to(DEV), small.kv.to(DEV), small.indices.to(DEV), small.sm_scale, small.d_v,
             attn_sink=sk)
    assert smla.last_kernel() == ("ring" if ring else "wide")
    del kv_big
    torch.cuda.empty_cache()


def test_decode_pool_past_4gib():
    c = W.make_decode("big_pool", batch=3, s_q=2, h_q=128, d_qk=576, d_v=512, topk=256,
                      seqlens=torch.tensor([900, 300, 2000]), seed=8, effective=200,
                      with_length=True, with_sink=True, spare_pages=4)
    big_pages = BIG_ROWS // 64
    gen = torch.Generator().manual_seed(9)
    n = c.kv_cache.shape[0]
    new_page = (big_pages - 1 - torch.randperm(big_pages // 4, generator=gen)[:n]).to(torch.int32)
    bt = c.block_table.clone()
    bt[bt >= 0] = new_page[bt[bt >= 0].long()]
    pool = torch.zeros((big_pages, 64, 1, 576), dtype=torch.bfloat16, device=DEV)
    pool[new_page.long().to(DEV)] = c.kv_cache.to(DEV)
    _say(c.name)
    t = lambda x: None if x is None else x.to(DEV)  # noqa: E731
    res = smla.decode_fwd(t(c.q), pool, t(bt), t(c.cache_seqlens), t(c.indices), c.sm_scale,
                          c.d_v, attn_sink=t(c.attn_sink), topk_length=t(c.topk_length))
    assert smla.last_kernel() == "ring_big"
    torch.cuda.synchronize()
    ref = oracle_decode(c)
    assert_parity(res, ref, c.name + " in a >4 GiB pool")
    # split decode over the same pool (the wide kernel's BIG form)
    res = smla.decode_fwd_split(t(c.q), pool, t(bt), t(c.cache_seqlens), t(c.indices), c.sm_scale,
                                3, c.d_v, attn_sink=t(c.attn_sink), topk_length=t(c.topk_length))
    assert smla.last_kernel() == "ring_split_big"
    torch.cuda.synchronize()
    assert_parity(res, ref, c.name + " split in a >4 GiB pool")
    del pool
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# randomized shapes: head counts, d_qk, row counts beyond the grid, lengths,
# sinks, paging and split counts drawn from a fixed seed
# ---------------------------------------------------------------------------

def _random_case(rng, i):
    h = rng.choice([64, 128, 64, 128, 16, 96]); d = rng.choice([512, 576])
    sink = rng.random() < 0.5
    seed = rng.randrange(1 << 20)
    if rng.random() < 0.6:
        s_kv = rng.choice([100, 700, 2000])
        topk = min(rng.choice([1, 31, 33, 64, 65, 96, 200, 256]), s_kv)
        lay = rng.choice(["scattered", "ramp"])
        kw = (dict(invalid_frac=rng.choice([0.0, 0.1, 0.5]), empty_frac=0.05)
              if lay == "scattered" else dict(ramp_cap=topk // 2 + 1))
        c = W.make_prefill(f"rnd{i}_h{h}_d{d}", s_q=rng.choice([3, 100, 300, 513]), s_kv=s_kv,
                           h_q=h, d_qk=d, d_v=512, topk=topk, layout=lay, seed=seed,
                           with_sink=sink, **kw)
        tl = None
        if rng.random() < 0.4:
            tl = torch.randint(0, topk + 1, (c.s_q,), dtype=torch.int32,
                               generator=torch.Generator().manual_seed(seed))
        return c, tl, 0
    B, s_q, topk = rng.choice([2, 40, 150]), rng.choice([1, 2, 3]), rng.choice([64, 128, 256])
    eff = rng.choice([topk, topk // 2])
    seqlens = torch.randint(eff, eff + 900, (B,), generator=torch.Generator().manual_seed(seed))
    c = W.make_decode(f"rnd{i}_dec_h{h}_d{d}", batch=B, s_q=s_q, h_q=h, d_qk=d, d_v=512,
                      topk=topk, seqlens=seqlens, seed=seed, effective=eff,
                      with_length=rng.random() < 0.5, with_sink=sink)
    split_ok = h == 128 or (h == 64 and d == 512)
    return c, None, rng.choice([1, 2, 5]) if split_ok else 1


def test_randomized_shapes():
    import random
    rng = random.Random(2024)
    for i in range(24):
        c, tl, splits = _random_case(rng, i)
        _say(f"{c.name} splits={splits}")
        if hasattr(c, "kv_cache"):
            got = run_decode_split(c, splits) if splits > 1 else run_decode(c)
            assert_parity(got, oracle_decode(c), c.name)
        else:
            got = run_prefill(c, topk_length=tl if tl is not None else "case")
            assert_parity(got, oracle_prefill(c, topk_length=tl if tl is not None else "case"),
                          c.name)


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times:
# sampled rows against the oracle, properties on every row
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def h64_full():
    c_nolen = W.prefill_h64(with_length=False)
    c_len = W.prefill_h64(with_length=True)
    assert torch.equal(c_nolen.indices, c_len.indices) and torch.equal(c_nolen.q, c_len.q)
    return c_nolen, c_len


def test_full_prefill_h64(h64_full):
    c_nolen, c_len = h64_full
    _say(c_nolen.name + " (full)")
    a = run_prefill(c_nolen)
    b = run_prefill(c_len)
    assert_bitwise(a, b, "full h64: derived vs explicit length")
    rows = sample_rows(c_nolen.s_q, 20, seed=0, must=(1, 63, 64, 1025, 1026, 1027, 4095))
    assert_parity(a, oracle_prefill(c_nolen, rows=rows), c_nolen.name, rows=rows)
    rl = smla.row_lengths(c_nolen.indices.to(DEV), s_kv=c_nolen.s_kv).cpu()
    assert torch.equal(rl, c_len.topk_length)
    assert torch.isfinite(a[1]).all() and torch.isfinite(a[0].float()).all()


def test_full_prefill_h128():
    c = W.prefill_h128()
    _say(c.name + " (full)")
    res = run_prefill(c)
    empty = c.meta["empty_rows"]
    rows = sample_rows(c.s_q, 14, seed=1, must=empty[:3])
    assert_parity(res, oracle_prefill(c, rows=rows), c.name, rows=rows)
    # every empty row of the workload is exact; every other row is finite
    lse = res[1].cpu()
    is_empty = torch.zeros(c.s_q, dtype=torch.bool)
    is_empty[empty] = True
    assert (lse[is_empty] == math.inf).all() and (res[0].cpu()[is_empty] == 0).all()
    assert torch.isfinite(lse[~is_empty]).all()
    rl = smla.row_lengths(c.indices.to(DEV), s_kv=c.s_kv).cpu().numpy()
    assert np.array_equal(rl, oracle.row_lengths(c.indices, s_kv=c.s_kv))
    # Every row: the derived lengths given explicitly change nothing, bit for bit.
    explicit = run_prefill(c, topk_length=torch.from_numpy(rl).to(torch.int32))
    assert_bitwise(res, explicit, "full h128: derived vs explicit length")


def test_full_decode_dynamic():
    c = W.decode_dynamic(with_length=True)
    _say(c.name + " (full)")
    dyn = run_decode(c)
    rows = sample_rows(c.batch, 12, seed=2)
    assert_parity(dyn, oracle_decode(c, rows=rows), c.name, rows=rows)
    fixed = W.decode_dynamic(with_length=False)
    assert_bitwise(dyn, run_decode(fixed), "full decode: fixed vs dynamic")


def test_full_decode_fixed():
    c = W.decode_fixed()
    _say(c.name + " (full)")
    res = run_decode(c)
    rows = sample_rows(c.batch * c.s_q, 12, seed=3)
    assert_parity(res, oracle_decode(c, rows=rows), c.name, rows=rows)
    assert torch.isfinite(res[0].float()).all() and torch.isfinite(res[1]).all()
    # Every row: lengths topk - (row % 64) given explicitly, against the same
    # positions past each length poisoned with INT_MAX (an invalid index) and
    # the length left to the tail scan; the two must agree bit for bit.
    B, s_q, topk = c.indices.shape
    lengths = (topk - torch.arange(B * s_q) % 64).to(torch.int32).view(B, s_q)
    poisoned = c.indices.clone()
    pos = torch.arange(topk).view(1, 1, topk)
    poisoned[pos >= lengths.unsqueeze(-1)] = 2**31 - 1
    explicit = run_decode(c, topk_length=lengths)
    derived = run_decode(c, topk_length=None, indices=poisoned)
    assert_bitwise(explicit, derived, "full decode: explicit lengths vs INT_MAX past them")
