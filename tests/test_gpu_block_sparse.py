"""GPU-vs-oracle parity of the block-sparse forward (sparse_mla_block_sparse_fwd).

Same bar as the sparse forward (tests/parity.py): out max-abs <= 2e-2 and
rel-L2 <= 1e-2, lse max-abs <= 1e-3; rows without keys give out = +0 and
lse = +inf exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_amd as smla
from parity import LSE_ABS, OUT_MAX_ABS, OUT_REL_L2, to_np64
from sparse_top_mla_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(case):
    print(f"[block-sparse] {case.name} s={case.s} h_q={case.h_q} h_kv={case.k.shape[1]} "
          f"q_block={case.q_block} k_block={case.k_block} causal={case.causal} "
          f"nnz={case.col_idx.numel()}", flush=True)
    out, lse = smla.block_sparse_fwd(case.q.to(DEV), case.k.to(DEV), case.v.to(DEV),
                                     case.row_ptr.to(DEV), case.col_idx.to(DEV), case.q_block,
                                     case.k_block, case.sm_scale, causal=case.causal)
    torch.cuda.synchronize()
    return out, lse


def _check(case, out, lse, rows=None):
    r_out, r_lse = oracle.block_sparse_fwd(case.q, case.k, case.v, case.row_ptr, case.col_idx,
                                           case.q_block, case.k_block, case.sm_scale,
                                           causal=case.causal, rows=rows)
    g_out, g_lse = to_np64(out), to_np64(lse)
    if rows is not None:
        g_out, g_lse = g_out[rows], g_lse[rows]
    empty = np.isinf(r_lse)
    if empty.any():
        assert np.all(g_lse[empty] == np.inf), "rows without keys give lse = +inf"
        eo = np.where(empty[:, :, None], g_out, 0.0)
        assert np.all(eo == 0.0) and not np.any(np.signbit(eo)), "rows without keys give out = +0"
    full = ~empty
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse[full]))
    max_abs = float(np.abs(g_out - r_out).max())
    denom = float(np.linalg.norm(r_out))
    rel_l2 = float(np.linalg.norm(g_out - r_out)) / denom if denom > 0 else 0.0
    lse_err = float(np.abs(g_lse[full] - r_lse[full]).max()) if full.any() else 0.0
    print(f"[block-sparse] {case.name}: out max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} "
          f"lse={lse_err:.3e} empty={int(empty.sum())}", flush=True)
    assert max_abs <= OUT_MAX_ABS and rel_l2 <= OUT_REL_L2 and lse_err <= LSE_ABS


@pytest.mark.parametrize("selection,causal", [("random", True), ("random", False),
                                              ("sink_window", True), ("sink_window", False),
                                              ("full_causal", True)])
@pytest.mark.parametrize("q_block,k_block", [(64, 64), (256, 128), (128, 192)])
def test_block_sparse_matches_oracle(selection, q_block, k_block, causal):
    case = W.make_block_sparse(f"bs_{selection}_q{q_block}_k{k_block}", s=700, h_q=4, h_kv=2,
                               q_block=q_block, k_block=k_block, selection=selection,
                               causal=causal, seed=q_block + k_block + causal)
    out, lse = _run(case)
    _check(case, out, lse)


def test_block_sparse_empty_selections_and_grouped_heads():
    """Query blocks with no selected block, only out-of-range ids, or a block
    listed twice; 8 query heads on 2 KV heads."""
    case = W.make_block_sparse("bs_edges", s=300, h_q=8, h_kv=2, q_block=64, k_block=64,
                               selection="random", seed=5)
    lists = [[], [-1, 9, 100], [0, 0, 1], [2, 3, 1, 0], [4]]
    ptr, col = W._csr(lists)
    case.row_ptr, case.col_idx = ptr, col
    out, lse = _run(case)
    _check(case, out, lse)
    assert torch.all(out[:128] == 0) and torch.all(torch.isinf(lse[:128]))


def test_block_sparse_full_size_sampled():
    """The pages' benchmark shape: s = 65536, h = 8, q_block 256, k_block
    128, key block 0 plus a 4-block window; sampled rows."""
    case = W.block_sparse_h8()
    out, lse = _run(case)
    rows = np.array([0, 1, 63, 64, 255, 256, 511, 1000, 4095, 30000, 65279, 65280, 65535])
    _check(case, out, lse, rows=rows)


def test_block_sparse_one_kv_head_not_causal():
    """16 query heads on one KV head, no causal mask, 128-row workgroups with
    a sequence that ends inside a workgroup and inside a key block."""
    case = W.make_block_sparse("bs_mqa_noncausal", s=1000, h_q=16, h_kv=1, q_block=128,
                               k_block=64, selection="random", causal=False, seed=21, density=0.5)
    out, lse = _run(case)
    _check(case, out, lse)


def test_block_sparse_random_shapes():
    """Seeded random shapes: sequence lengths down to 1, head groupings, both
    workgroup sizes (query blocks multiple of 128 or only of 64), key blocks
    of 64 to 192, causal or not, random selections."""
    rng = np.random.default_rng(77)
    for t in range(10):
        s = int(rng.choice([1, 7, 63, 64, 65, 200, 513, 900]))
        h_kv = int(rng.choice([1, 2, 4]))
        h_q = h_kv * int(rng.choice([1, 2, 4]))
        q_block = int(rng.choice([64, 128, 192, 256]))
        k_block = int(rng.choice([64, 128, 192]))
        causal = bool(rng.integers(0, 2))
        case = W.make_block_sparse(f"bs_rand{t}_s{s}_h{h_q}x{h_kv}_q{q_block}_k{k_block}", s=s,
                                   h_q=h_q, h_kv=h_kv, q_block=q_block, k_block=k_block,
                                   selection="random", causal=causal, seed=100 + t,
                                   density=float(rng.uniform(0.2, 0.9)))
        out, lse = _run(case)
        _check(case, out, lse)
