"""GPU-vs-oracle parity of the sparse MLA backward (sparse_mla_bwd).

The backward's inputs besides q, kv, indices are the forward's out and lse
and the gradient dout.  Small cases take out and lse from the oracle's own
forward (rounded to the bf16 / fp32 the library receives); the full-size case
takes seeded stand-ins of the same size (the oracle forward over 4096 rows x
2048 keys is too slow for a test), since the backward is a formula in those
inputs.  Both sides always receive the same values.

Tolerances (fp32 accumulation, bf16 P, dS and outputs; the oracle is fp64):
relative L2 error <= 1e-2 and max-abs error <= 2e-2 of the largest reference
magnitude, for dq, dkv and d_sink.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_top_mla_amd as smla
from sparse_top_mla_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REL_L2 = 1e-2
MAX_REL = 2e-2


def _t(x):
    return None if x is None else x.to(DEV)


def _close(name, got, ref):
    g = got.detach().float().cpu().double().numpy() if isinstance(got, torch.Tensor) else got
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    scale = np.abs(r).max()
    if scale == 0.0:
        assert np.all(g == 0.0), f"{name}: expected zeros, max |got| {np.abs(g).max():.3e}"
        return
    err = np.abs(g - r)
    rel_l2 = np.linalg.norm(g - r) / np.linalg.norm(r)
    max_rel = err.max() / scale
    print(f"[bwd] {name}: rel_l2 {rel_l2:.2e} max_abs/scale {max_rel:.2e} (scale {scale:.3e})",
          flush=True)
    assert rel_l2 <= REL_L2 and max_rel <= MAX_REL, \
        f"{name}: rel_l2 {rel_l2:.3e} max_abs/scale {max_rel:.3e}"


def _oracle_stats(case):
    """The oracle forward's out (bf16) and lse (fp32)."""
    out, lse, _, _ = oracle.sparse_mla_fwd(case.q, case.kv, case.indices, case.sm_scale, case.d_v,
                                           attn_sink=case.attn_sink, topk_length=case.topk_length)
    return torch.from_numpy(out).to(torch.bfloat16), torch.from_numpy(lse).to(torch.float32)


def _run(case, out, lse, dout, lse_base2=False, with_d_sink=None):
    with_d_sink = case.attn_sink is not None if with_d_sink is None else with_d_sink
    lse_in = lse / math.log(2.0) if lse_base2 else lse
    print(f"[bwd] {case.name} s_q={case.s_q} s_kv={case.s_kv} topk={case.topk} "
          f"d_qk={case.d_qk} sink={case.attn_sink is not None} "
          f"len={case.topk_length is not None} base2={lse_base2}", flush=True)
    dq, dkv, ds = smla.bwd(_t(case.q), _t(case.kv), _t(out), _t(dout), _t(case.indices),
                           _t(lse_in.to(torch.float32)), case.sm_scale, case.d_v,
                           attn_sink=_t(case.attn_sink), topk_length=_t(case.topk_length),
                           lse_base2=lse_base2, want_d_sink=with_d_sink)
    torch.cuda.synchronize()
    return dq, dkv, ds


def _small(d_qk, with_length, with_sink, seed, s_q=48, s_kv=200, topk=96):
    if with_length:
        case = W.make_prefill(f"bwd_small_ramp_d{d_qk}", s_q=s_q, s_kv=s_kv, h_q=64, d_qk=d_qk,
                              d_v=512, topk=topk, layout="ramp", ramp_cap=topk - 7, seed=seed,
                              with_length=True, with_sink=with_sink)
    else:
        case = W.make_prefill(f"bwd_small_scatter_d{d_qk}", s_q=s_q, s_kv=s_kv, h_q=64,
                              d_qk=d_qk, d_v=512, topk=topk, layout="scattered",
                              invalid_frac=0.1, empty_frac=0.05, with_sink=with_sink, seed=seed)
        # A key named twice in one row (two atomics of one workgroup on one KV row).
        case.indices[1, 0, 5] = case.indices[1, 0, 2]
        case.indices[1, 0, 40] = case.indices[1, 0, 2]
    return case


@pytest.mark.parametrize("d_qk", [576, 512])
@pytest.mark.parametrize("with_length,with_sink", [(False, False), (True, False), (False, True),
                                                   (True, True)])
def test_bwd_matches_oracle(d_qk, with_length, with_sink):
    case = _small(d_qk, with_length, with_sink, seed=11 + d_qk + 2 * with_length + with_sink)
    dout = W.bwd_dout(case, seed=5)
    out, lse = _oracle_stats(case)
    dq, dkv, ds = _run(case, out, lse, dout)
    # s_kv = 200 is within 4 row widths of topk = 96: the key-outer dkv pass,
    # with row 1 of the unlengthed case (a key named three times) scattered
    # by the row pass.
    assert smla.last_kernel() == "bwd_key_outer"
    rq, rkv, rs = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                        case.sm_scale, case.d_v, attn_sink=case.attn_sink,
                                        topk_length=case.topk_length,
                                        want_d_sink=with_sink)
    _close("dq", dq, rq)
    _close("dkv", dkv[:, 0, :], rkv)
    if with_sink:
        _close("d_sink", ds, rs)


def test_bwd_lse_base2():
    case = _small(576, False, True, seed=31)
    dout = W.bwd_dout(case, seed=6)
    out, lse = _oracle_stats(case)
    dq, dkv, ds = _run(case, out, lse, dout, lse_base2=True)
    dq0, dkv0, ds0 = _run(case, out, lse, dout)
    rq, rkv, rs = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                        case.sm_scale, case.d_v, attn_sink=case.attn_sink,
                                        want_d_sink=True)
    _close("dq (base-2 lse)", dq, rq)
    _close("dkv (base-2 lse)", dkv[:, 0, :], rkv)
    _close("d_sink (base-2 lse)", ds, rs)
    # The same normaliser in either base: both runs agree to fp32 rounding of lse.
    _close("dq base-2 vs natural", dq, dq0.float().cpu().double().numpy())


def test_bwd_tails_empty_rows_and_unnamed_kv_rows():
    """topk not a multiple of the 32-key block, rows of length 0, 1, 31, 32,
    33, and KV rows no query names (their dkv is exactly 0)."""
    case = W.make_prefill("bwd_tails_d576", s_q=8, s_kv=120, h_q=64, d_qk=576, d_v=512, topk=70,
                          layout="full", seed=41)
    idx = case.indices.view(8, 70)
    idx[idx >= 100] = 3  # rows 100..119 are never named
    lengths = torch.tensor([0, 1, 31, 32, 33, 70, 64, 65], dtype=torch.int32)
    case.topk_length = lengths
    dout = W.bwd_dout(case, seed=7)
    out, lse = _oracle_stats(case)
    dq, dkv, _ = _run(case, out, lse, dout)
    rq, rkv, _ = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                       case.sm_scale, case.d_v, topk_length=lengths)
    _close("dq", dq, rq)
    _close("dkv", dkv[:, 0, :], rkv)
    assert torch.all(dq[0] == 0), "a row without keys has dq = 0"
    assert torch.all(dkv[100:] == 0), "KV rows no query names have dkv = 0"


def test_bwd_full_size_sampled():
    """T = 4096, topk = 2048, h_q = 64, d_qk = 576 (the pages' backward shape):
    dq of sampled rows and dkv of sampled KV rows against the oracle."""
    case = W.bwd_h64()
    dout = W.bwd_dout(case, seed=8)
    out, lse = W.bwd_synthetic_stats(case, seed=9)
    dq, dkv, _ = _run(case, out, lse, dout)
    assert smla.last_kernel() == "bwd_key_outer"
    rows = np.array([0, 1, 31, 32, 1023, 2047, 2048, 2049, 3000, 4094, 4095])
    kv_rows = np.array([0, 1, 17, 640, 2047, 2048, 3071, 4000, 4095])
    rq, rkv, _ = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                       case.sm_scale, case.d_v, topk_length=case.topk_length,
                                       rows=rows, kv_rows=kv_rows)
    _close("dq (sampled rows)", dq[torch.from_numpy(rows).to(DEV)], rq)
    _close("dkv (sampled KV rows)", dkv[torch.from_numpy(kv_rows).to(DEV), 0, :], rkv)


def test_bwd_unsupported_heads_raise():
    case = W.make_prefill("bwd_h32", s_q=4, s_kv=64, h_q=32, d_qk=576, d_v=512, topk=32,
                          layout="full", seed=3)
    dout = W.bwd_dout(case, seed=1)
    out = torch.zeros(4, 32, 512, dtype=torch.bfloat16)
    lse = torch.zeros(4, 32)
    with pytest.raises(smla.SparseMLAError, match="h_q"):
        _run(case, out, lse, dout)


def test_bwd_d512_sampled():
    """d_qk = 512 at T = 2048, topk = 1024: dq of sampled rows and dkv of
    sampled KV rows."""
    case = W.bwd_h64(s_q=2048, s_kv=2048, topk=1024, d_qk=512)
    dout = W.bwd_dout(case, seed=12)
    out, lse = W.bwd_synthetic_stats(case, seed=13)
    dq, dkv, _ = _run(case, out, lse, dout)
    rows = np.array([0, 5, 1023, 1024, 1500, 2047])
    kv_rows = np.array([0, 3, 1000, 1024, 2040, 2047])
    rq, rkv, _ = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                       case.sm_scale, case.d_v, topk_length=case.topk_length,
                                       rows=rows, kv_rows=kv_rows)
    _close("dq (sampled rows, d512)", dq[torch.from_numpy(rows).to(DEV)], rq)
    _close("dkv (sampled KV rows, d512)", dkv[torch.from_numpy(kv_rows).to(DEV), 0, :], rkv)


def test_bwd_random_shapes():
    """Seeded random shapes: row and KV counts, topk not a multiple of the
    32-key block, d_qk, layout, lengths and sink."""
    rng = np.random.default_rng(91)
    for t in range(6):
        d_qk = int(rng.choice([512, 576]))
        s_q = int(rng.integers(1, 40))
        s_kv = int(rng.integers(8, 300))
        topk = int(rng.integers(1, min(s_kv, 130) + 1))
        layout = str(rng.choice(["ramp", "scattered"]))
        sink = bool(rng.integers(0, 2))
        kw = dict(ramp_cap=topk, with_length=bool(rng.integers(0, 2))) if layout == "ramp" else \
            dict(invalid_frac=0.2, empty_frac=0.1)
        case = W.make_prefill(f"bwd_rand{t}_d{d_qk}_{layout}", s_q=s_q, s_kv=s_kv, h_q=64,
                              d_qk=d_qk, d_v=512, topk=topk, layout=layout, seed=200 + t,
                              with_sink=sink, **kw)
        dout = W.bwd_dout(case, seed=300 + t)
        out, lse = _oracle_stats(case)
        dq, dkv, ds = _run(case, out, lse, dout)
        rq, rkv, rs = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                            case.sm_scale, case.d_v, attn_sink=case.attn_sink,
                                            topk_length=case.topk_length, want_d_sink=sink)
        _close(f"dq {case.name}", dq, rq)
        _close(f"dkv {case.name}", dkv[:, 0, :], rkv)
        if sink:
            _close(f"d_sink {case.name}", ds, rs)


@pytest.mark.parametrize("d_qk", [576, 512])
def test_bwd_key_outer_and_scatter_paths_agree(d_qk):
    """One selection through both dkv paths: topk = 40 over s_kv = 400 KV rows
    scatters per (row, key) pair (the table is more than 4 row widths), and
    the same indices padded with -1 to topk = 100 go through the key-outer
    pass.  Both match the oracle; ragged key blocks (400 = 6 x 64 + 16) and
    a ragged last row chunk (s_q = 150) included."""
    case = W.make_prefill(f"bwd_paths_d{d_qk}", s_q=150, s_kv=400, h_q=64, d_qk=d_qk, d_v=512,
                          topk=40, layout="scattered", invalid_frac=0.1, empty_frac=0.05,
                          seed=77, with_sink=True)
    dout = W.bwd_dout(case, seed=78)
    out, lse = _oracle_stats(case)
    dq_s, dkv_s, ds_s = _run(case, out, lse, dout)
    assert smla.last_kernel() == "bwd_scatter"
    padded = torch.full((150, 1, 100), -1, dtype=torch.int32)
    padded[:, :, :40] = case.indices
    wide = dataclasses.replace(case, name=case.name + "_padded", indices=padded)
    dq_k, dkv_k, ds_k = _run(wide, out, lse, dout)
    assert smla.last_kernel() == "bwd_key_outer"
    rq, rkv, rs = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                        case.sm_scale, case.d_v, attn_sink=case.attn_sink,
                                        want_d_sink=True)
    for tag, dq, dkv, ds in (("scatter", dq_s, dkv_s, ds_s), ("key-outer", dq_k, dkv_k, ds_k)):
        _close(f"dq ({tag})", dq, rq)
        _close(f"dkv ({tag})", dkv[:, 0, :], rkv)
        _close(f"d_sink ({tag})", ds, rs)
    # dq comes from the same per-row sums on both paths (d_sink's cross-row
    # atomic sum has a run-dependent order).
    assert torch.equal(dq_s, dq_k)


def test_bwd_key_outer_with_wide_rows():
    """topk = 3200 (above the dq pass's 3072-entry index list) over s_kv = 4000:
    a key-outer call whose dq comes from the row pass itself, with a row that
    names a key twice among them."""
    case = W.make_prefill("bwd_wide_rows_d576", s_q=6, s_kv=4000, h_q=64, d_qk=576, d_v=512,
                          topk=3200, layout="scattered", invalid_frac=0.1, empty_frac=0.0,
                          seed=97, with_sink=True)
    case.indices[2, 0, 3000] = case.indices[2, 0, 17]
    dout = W.bwd_dout(case, seed=98)
    out, lse = _oracle_stats(case)
    dq, dkv, ds = _run(case, out, lse, dout)
    assert smla.last_kernel() == "bwd_key_outer"
    rq, rkv, rs = oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse,
                                        case.sm_scale, case.d_v, attn_sink=case.attn_sink,
                                        want_d_sink=True)
    _close("dq (wide rows)", dq, rq)
    _close("dkv (wide rows)", dkv[:, 0, :], rkv)
    _close("d_sink (wide rows)", ds, rs)
