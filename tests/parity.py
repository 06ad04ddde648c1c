"""Comparison of the HIP path against the fp64 CPU oracle.

Tolerances (bf16 inputs; fp32 accumulation on the GPU, fp64 in the oracle):
  out         max |gpu - oracle| <= 2e-2  and  ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2
  lse         max |gpu - oracle| <= 1e-3   (finite entries)
  max_logits  max |gpu - oracle| <= 1e-3   (finite entries)
  rows without a key: out == +0 exactly, lse == +inf, max_logits == -inf
  row lengths: bit-exact
"""
from __future__ import annotations

import numpy as np
import torch

OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 1e-2
LSE_ABS = 1e-3
MAX_LOGITS_ABS = 1e-3


def to_np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(gpu, ref, name="", rows=None):
    """gpu = (out, lse, max_logits) torch tensors; ref = oracle tuple (out, lse,
    max_logits, ...) in fp64 for the rows `rows` (all rows when None)."""
    g_out, g_lse, g_ml = gpu
    h_q, d_v = g_out.shape[-2], g_out.shape[-1]
    g_out = to_np64(g_out).reshape(-1, h_q, d_v)
    g_lse = to_np64(g_lse).reshape(-1, h_q)
    g_ml = to_np64(g_ml).reshape(-1, h_q)
    if rows is not None:
        rows = np.asarray(rows)
        g_out, g_lse, g_ml = g_out[rows], g_lse[rows], g_ml[rows]
    r_out, r_lse, r_ml = ref[0], ref[1], ref[2]
    assert g_out.shape == r_out.shape, (g_out.shape, r_out.shape)

    empty = np.isinf(r_lse)
    assert np.all(r_lse[empty] > 0) and np.all(r_ml[empty] == -np.inf)
    if empty.any():
        assert np.all(g_lse[empty] == np.inf), f"{name}: empty rows must give lse=+inf"
        assert np.all(g_ml[empty] == -np.inf), f"{name}: empty rows must give max_logits=-inf"
        eo = g_out[empty]
        assert np.all(eo == 0.0) and not np.any(np.signbit(eo)), f"{name}: empty rows must give out=+0"
    full = ~empty
    assert np.all(np.isfinite(g_lse[full])), f"{name}: non-finite lse on a row with keys"
    assert np.all(np.isfinite(g_ml[full])), f"{name}: non-finite max_logits on a row with keys"
    assert np.all(np.isfinite(g_out)), f"{name}: non-finite out"

    err = np.abs(g_out - r_out)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(r_out))
    rel_l2 = float(np.linalg.norm(g_out - r_out)) / denom if denom > 0 else 0.0
    lse_err = float(np.abs(g_lse[full] - r_lse[full]).max()) if full.any() else 0.0
    ml_err = float(np.abs(g_ml[full] - r_ml[full]).max()) if full.any() else 0.0
    print(f"[parity] {name}: out max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} "
          f"lse={lse_err:.3e} max_logits={ml_err:.3e} empty={int(empty.sum())}", flush=True)
    assert max_abs <= OUT_MAX_ABS, f"{name}: out max_abs {max_abs:.3e}"
    assert rel_l2 <= OUT_REL_L2, f"{name}: out rel_l2 {rel_l2:.3e}"
    assert lse_err <= LSE_ABS, f"{name}: lse err {lse_err:.3e}"
    assert ml_err <= MAX_LOGITS_ABS, f"{name}: max_logits err {ml_err:.3e}"
    return dict(max_abs=max_abs, rel_l2=rel_l2, lse=lse_err, max_logits=ml_err)


def assert_bitwise(a, b, name=""):
    for x, y, what in zip(a, b, ("out", "lse", "max_logits")):
        assert torch.equal(x, y), f"{name}: {what} differs bitwise"


def sample_rows(n_rows, k, seed, must=()):
    gen = np.random.default_rng(seed)
    picks = set(int(r) for r in must if 0 <= r < n_rows)
    picks.update([0, n_rows - 1])
    if n_rows > 2:
        picks.update(gen.choice(n_rows, size=min(k, n_rows), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
