"""Pins that tie the CPU oracle to something other than itself.

Each pin takes an oracle library handle (``oracle.load()`` or a library built
from a deliberately broken copy of the oracle source) and raises
AssertionError when the oracle disagrees with:

  * a library routine on a special case of the method (dense multi-query
    softmax attention via torch's scaled_dot_product_attention in float64,
    with the attention sink as an extra value-less key carried by an additive
    mask -- the "sink-column reference" of FlashMLA PR #198, "Numerics");
  * a differently formulated brute force (dense attention over every KV row
    with additive bias ln(multiplicity), in numpy float64);
  * closed forms (single key, a key repeated k times, the sink as a logistic
    factor, max_logits <= lse <= max_logits + ln |keys|);
  * the fixed conventions of the pages (empty row -> 0, +inf, -inf, FlashMLA
    PR #196 "Correctness notes"; row lengths of tests/golden/row_lengths.txt);
  * invariances the pages state (derived == explicit length, PR #196
    "Numbers"; INT_MAX-poisoned dynamic == -1-padded fixed, PR #216
    "Dynamic top-k"; any invalid encoding masks alike, PR #196 "Fix");
  * for the backward (PR #198, "Summary", item 1): float64 autograd of the
    dense multiplicity-bias attention (with the sink as an extra value-less
    column, PR #198 "Numerics"), a single-key closed form, base-2 lse
    (PR #198's bwd contract) and row / KV-row selection;
  * for the block-sparse forward (PR #198, "Summary", item 3, "Benchmarks":
    a full-causal selection reproduces dense attention): torch SDPA in
    float64 for full causal and full non-causal selections (with grouped KV
    heads), and a numpy dense-mask brute force for random selections.

tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py checks that each planted mistake fails one.
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import torch

import oracle

GOLDEN = Path(__file__).resolve().parent / "golden"
INT32_MAX = 2**31 - 1


# ---------------------------------------------------------------------------
# tiny seeded inputs for the pins
# ---------------------------------------------------------------------------

def _bf16(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16)


def _f64(t):
    return t.to(torch.float64)


def _tiny(seed, s_q=5, s_kv=37, h_q=4, d_qk=24, d_v=16):
    gen = torch.Generator().manual_seed(seed)
    q = _bf16((s_q, h_q, d_qk), gen)
    kv = _bf16((s_kv, 1, d_qk), gen)
    return gen, q, kv


def _multiplicity_reference(q, kv, indices, sm_scale, d_v, topk_length=None, sink=None):
    """Dense attention over all s_kv rows with bias ln(count), count being how
    often a row is named at a position before the row's length.  Everything in
    numpy float64."""
    qn = _f64(q).numpy()
    kvn = _f64(kv[:, 0, :]).numpy()
    idx = indices.reshape(indices.shape[0], -1).numpy().astype(np.int64)
    s_q, h_q, _ = qn.shape
    s_kv = kvn.shape[0]
    topk = idx.shape[1]
    out = np.zeros((s_q, h_q, d_v))
    lse = np.full((s_q, h_q), np.inf)
    ml = np.full((s_q, h_q), -np.inf)
    lens = np.zeros(s_q, dtype=np.int64)
    for r in range(s_q):
        valid = (idx[r] >= 0) & (idx[r] < s_kv)
        if topk_length is None:
            nz = np.nonzero(valid)[0]
            L = int(nz[-1]) + 1 if nz.size else 0
        else:
            L = int(min(max(int(topk_length[r]), 0), topk))
        lens[r] = L
        count = np.bincount(idx[r, :L][valid[:L]], minlength=s_kv).astype(np.float64)
        if count.sum() == 0:
            continue
        with np.errstate(divide="ignore"):
            bias = np.log(count)
        scores = sm_scale * (qn[r] @ kvn.T) + bias[None, :]  # [h_q, s_kv]
        m = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - m)
        Z = w.sum(axis=1)
        denom = Z + (np.exp(sink.numpy().astype(np.float64) - m[:, 0]) if sink is not None else 0.0)
        out[r] = (w @ kvn[:, :d_v]) / denom[:, None]
        lse[r] = m[:, 0] + np.log(Z)
        named = count > 0
        ml[r] = (sm_scale * (qn[r] @ kvn.T))[:, named].max(axis=1)
    return out, lse, ml, lens


def _close(a, b, rtol=1e-11, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    fa, fb = np.where(same_inf, 0.0, a), np.where(same_inf, 0.0, b)
    assert np.all(np.isfinite(fa) == np.isfinite(fb)), f"{what}: finiteness differs"
    err = np.abs(fa - fb)
    lim = atol + rtol * np.abs(fb)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e} (worst excess {(err - lim).max():.3e})"


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_dense_equals_library_attention(lib):
    """topk = s_kv with every row naming every key (in a random order) is plain
    multi-query softmax attention; compare with torch SDPA in float64."""
    for seed, (s_q, s_kv, h_q, d_qk, d_v) in enumerate([(5, 37, 4, 24, 16), (3, 64, 2, 40, 40),
                                                        (2, 70, 3, 16, 8)]):
        gen, q, kv = _tiny(100 + seed, s_q, s_kv, h_q, d_qk, d_v)
        perm = torch.stack([torch.randperm(s_kv, generator=gen) for _ in range(s_q)])
        indices = perm.to(torch.int32).view(s_q, 1, s_kv)
        scale = 0.7 / math.sqrt(d_qk)
        out, lse, ml, rl = oracle.sparse_mla_fwd(q, kv, indices, scale, d_v, lib=lib)
        qq = _f64(q).unsqueeze(2)  # [s_q, h_q, 1, d_qk]
        kk = _f64(kv[:, 0]).expand(s_q, h_q, s_kv, d_qk)
        vv = _f64(kv[:, 0, :d_v]).expand(s_q, h_q, s_kv, d_v)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)[:, :, 0]
        _close(out, ref.numpy(), what="dense out vs SDPA")
        scores = torch.einsum("shd,kd->shk", _f64(q), _f64(kv[:, 0]))
        scores = (scores * scale).numpy()
        from scipy.special import logsumexp
        _close(lse, logsumexp(scores, axis=-1), what="dense lse vs logsumexp")
        _close(ml, scores.max(axis=-1), what="dense max_logits")
        assert np.all(rl == s_kv)


def pin_sink_equals_extra_key(lib):
    """The sink as a value-less key: an extra all-zero KV row whose logit is
    set to sink[h] through an additive attention mask (SDPA, float64).  lse and
    max_logits are the sink-free ones."""
    s_q, s_kv, h_q, d_qk, d_v = 4, 29, 5, 32, 24
    gen, q, kv = _tiny(7, s_q, s_kv, h_q, d_qk, d_v)
    sink = torch.randn(h_q, generator=gen) * 2.0
    indices = torch.stack([torch.randperm(s_kv, generator=gen) for _ in range(s_q)])
    indices = indices.to(torch.int32).view(s_q, 1, s_kv)
    scale = 1.0 / math.sqrt(d_qk)
    out, lse, ml, _ = oracle.sparse_mla_fwd(q, kv, indices, scale, d_v, attn_sink=sink, lib=lib)
    out0, lse0, ml0, _ = oracle.sparse_mla_fwd(q, kv, indices, scale, d_v, lib=lib)
    k_ext = torch.cat([_f64(kv[:, 0]), torch.zeros(1, d_qk, dtype=torch.float64)])
    v_ext = torch.cat([_f64(kv[:, 0, :d_v]), torch.zeros(1, d_v, dtype=torch.float64)])
    mask = torch.zeros(h_q, 1, s_kv + 1, dtype=torch.float64)
    mask[:, 0, s_kv] = _f64(sink)
    ref = torch.nn.functional.scaled_dot_product_attention(
        _f64(q).unsqueeze(2), k_ext.expand(s_q, h_q, s_kv + 1, d_qk),
        v_ext.expand(s_q, h_q, s_kv + 1, d_v), attn_mask=mask, scale=scale)[:, :, 0]
    _close(out, ref.numpy(), what="sink out vs extra-key SDPA")
    _close(lse, lse0, rtol=0, atol=0, what="lse is sink-free")
    _close(ml, ml0, rtol=0, atol=0, what="max_logits is sink-free")


def pin_sink_closed_form(lib):
    """out_sink = out_nosink * sigmoid(lse - sink) per head; sink = -inf is
    exactly no sink."""
    gen, q, kv = _tiny(11, 6, 41, 3, 20, 12)
    idx = torch.randint(-3, 45, (6, 1, 30), generator=gen).to(torch.int32)
    sink = torch.randn(3, generator=gen)
    scale = 0.21
    o1, l1, m1, _ = oracle.sparse_mla_fwd(q, kv, idx, scale, 12, attn_sink=sink, lib=lib)
    o0, l0, m0, _ = oracle.sparse_mla_fwd(q, kv, idx, scale, 12, lib=lib)
    sig = 1.0 / (1.0 + np.exp(sink.numpy().astype(np.float64)[None, :] - l0))
    _close(o1, o0 * sig[:, :, None], what="sink logistic factor")
    _close(l1, l0, rtol=0, atol=0, what="lse unchanged by sink")
    _close(m1, m0, rtol=0, atol=0, what="max_logits unchanged by sink")
    neg = torch.full((3,), -math.inf)
    on, ln_, mn, _ = oracle.sparse_mla_fwd(q, kv, idx, scale, 12, attn_sink=neg, lib=lib)
    assert np.array_equal(on, o0) and np.array_equal(ln_, l0) and np.array_equal(mn, m0)


def pin_multiplicity_bruteforce(lib):
    """Random tiny rows with duplicates, every invalid encoding, and random
    explicit lengths, against the dense ln(count)-bias formulation."""
    for seed in range(4):
        s_q, s_kv, h_q, d_qk, d_v, topk = 9, 23, 3, 16, 10, 40
        gen, q, kv = _tiny(200 + seed, s_q, s_kv, h_q, d_qk, d_v)
        idx = torch.randint(0, s_kv, (s_q, topk), generator=gen)
        kinds = torch.randint(0, 6, (s_q, topk), generator=gen)
        idx = torch.where(kinds == 0, torch.full_like(idx, -1), idx)
        idx = torch.where(kinds == 1, torch.full_like(idx, s_kv), idx)
        idx = torch.where(kinds == 2, torch.full_like(idx, INT32_MAX), idx)
        idx[0] = -1  # empty row
        idx[1, 5:] = -4  # short row, trailing invalids
        idx = idx.to(torch.int32).view(s_q, 1, topk)
        sink = torch.randn(h_q, generator=gen) if seed % 2 else None
        scale = 1.0 / math.sqrt(d_qk)
        tl = None
        if seed >= 2:
            tl = torch.randint(-2, topk + 5, (s_q,), generator=gen).to(torch.int32)
        out, lse, ml, rl = oracle.sparse_mla_fwd(q, kv, idx, scale, d_v, attn_sink=sink,
                                                 topk_length=tl, lib=lib)
        r_out, r_lse, r_ml, r_len = _multiplicity_reference(q, kv, idx, scale, d_v,
                                                            topk_length=tl, sink=sink)
        assert np.array_equal(rl, r_len), "row lengths"
        _close(out, r_out, rtol=1e-10, atol=1e-12, what="bruteforce out")
        _close(lse, r_lse, rtol=1e-11, atol=1e-12, what="bruteforce lse")
        _close(ml, r_ml, rtol=1e-11, atol=1e-12, what="bruteforce max_logits")


def pin_closed_forms(lib):
    """One key: out is that key's value exactly and lse == max_logits.  The
    same key k times: out is the value, lse = max_logits + ln k.  Always
    max_logits <= lse <= max_logits + ln |keys|, and without a sink each out
    coordinate lies between the smallest and largest value of the keys."""
    gen, q, kv = _tiny(31, 6, 50, 4, 32, 20)
    one = torch.full((6, 1, 8), -1, dtype=torch.int32)
    picks = torch.randint(0, 50, (6,), generator=gen).to(torch.int32)
    one[:, 0, 3] = picks
    o1, l1, m1, r1 = oracle.sparse_mla_fwd(q, kv, one, 0.3, 20, lib=lib)
    vals = _f64(kv[picks.long(), 0, :20]).numpy()
    assert np.array_equal(o1, np.broadcast_to(vals[:, None, :], o1.shape)), "single key value"
    assert np.array_equal(l1, m1), "single key lse == max_logits"
    assert np.all(r1 == 4)
    for k in (2, 5, 8):
        rep = torch.full((6, 1, 8), -1, dtype=torch.int32)
        rep[:, 0, :k] = picks[:, None]
        ok, lk, mk, _ = oracle.sparse_mla_fwd(q, kv, rep, 0.3, 20, lib=lib)
        _close(ok, np.broadcast_to(vals[:, None, :], ok.shape), rtol=1e-15, atol=0, what="repeat out")
        _close(mk, m1, rtol=0, atol=0, what="repeat max_logits")
        _close(lk, m1 + math.log(k), rtol=1e-14, atol=1e-14, what="repeat lse = s + ln k")
    idx = torch.stack([torch.randperm(50, generator=gen)[:30] for _ in range(6)]).to(torch.int32)
    o, l, m, _ = oracle.sparse_mla_fwd(q, kv, idx.view(6, 1, 30), 0.3, 20, lib=lib)
    assert np.all(m <= l) and np.all(l <= m + math.log(30) + 1e-12), "lse bounds"
    for r in range(6):
        v = _f64(kv[idx[r].long(), 0, :20]).numpy()
        assert np.all(o[r] >= v.min(axis=0) - 1e-12) and np.all(o[r] <= v.max(axis=0) + 1e-12)


def pin_empty_rows(lib):
    """No valid key (all invalid, explicit length 0, or valid keys only past
    an explicit length) gives out = +0, lse = +inf, max_logits = -inf, with or
    without a sink."""
    gen, q, kv = _tiny(41, 4, 16, 3, 16, 8)
    idx = torch.full((4, 1, 70), -1, dtype=torch.int32)
    idx[1, 0, :] = 16
    idx[1, 0, 5] = INT32_MAX
    idx[2, 0, 10] = 3
    idx[3, 0, 0] = 5
    tl = torch.tensor([70, 70, 5, 0], dtype=torch.int32)
    for sink in (None, torch.randn(3, generator=gen)):
        for length in (None, tl):
            out, lse, ml, rl = oracle.sparse_mla_fwd(q, kv, idx, 0.25, 8, attn_sink=sink,
                                                     topk_length=length, lib=lib)
            rows = [0, 1] if length is None else [0, 1, 2, 3]
            for r in rows:
                assert np.all(out[r] == 0.0) and not np.any(np.signbit(out[r])), "empty out"
                assert np.all(lse[r] == np.inf), "empty lse"
                assert np.all(ml[r] == -np.inf), "empty max_logits"
            if length is None:
                assert list(rl) == [0, 0, 11, 1]
            else:
                assert list(rl) == [70, 70, 5, 0]


def _golden_rows():
    rows = []
    for line in (GOLDEN / "row_lengths.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, topk, s_kv, explicit, exp_len, exp_blocks, fill, valid = line.split()
        topk, s_kv, exp_len, exp_blocks, fill = int(topk), int(s_kv), int(exp_len), int(exp_blocks), int(fill)
        row = np.full(topk, fill, dtype=np.int64)
        if valid != "-":
            for item in valid.split(","):
                p, v = item.split("=")
                row[int(p)] = int(v)
        rows.append((name, row.astype(np.int32), s_kv, None if explicit == "-" else int(explicit),
                     exp_len, exp_blocks))
    return rows


def pin_row_length_fixtures(lib):
    for name, row, s_kv, explicit, exp_len, exp_blocks in _golden_rows():
        tl = None if explicit is None else np.array([explicit], dtype=np.int32)
        got = oracle.row_lengths(row.reshape(1, -1), tl, s_kv=s_kv, lib=lib)[0]
        assert got == exp_len, f"{name}: L={got}, expected {exp_len}"
        assert max(-(-got // 64), 1) == exp_blocks, name
        # the paged form with the same bound gives the same length
        cs = np.array([s_kv], dtype=np.int32)
        got2 = oracle.row_lengths(row.reshape(1, -1), tl, cs, addressable=1 << 40, lib=lib)[0]
        assert got2 == exp_len, f"{name} (paged bound)"


def pin_row_length_bruteforce(lib):
    gen = torch.Generator().manual_seed(5)
    for topk in (1, 7, 64, 65, 200):
        idx = torch.randint(-5, 40, (50, topk), generator=gen)
        idx[::7] = -1
        idx[3::11] = INT32_MAX
        n = idx.numpy()
        got = oracle.row_lengths(n.astype(np.int32), s_kv=33, lib=lib)
        for r in range(50):
            v = np.nonzero((n[r] >= 0) & (n[r] < 33))[0]
            assert got[r] == (v[-1] + 1 if v.size else 0)
        seqlens = torch.randint(-3, 60, (10,), generator=gen).to(torch.int32)
        got = oracle.row_lengths(n.astype(np.int32), None, seqlens, rows_per_seq=5,
                                 addressable=40, lib=lib)
        for r in range(50):
            bound = min(int(seqlens[r // 5]), 40)
            v = np.nonzero((n[r] >= 0) & (n[r] < bound))[0]
            assert got[r] == (v[-1] + 1 if v.size else 0)


def pin_length_and_encoding_invariance(lib):
    """Derived length == explicit length equal to it (bitwise); -1 padding
    without a length == INT_MAX poisoning with a length (bitwise); swapping one
    invalid encoding for another changes nothing (bitwise)."""
    gen, q, kv = _tiny(51, 8, 40, 3, 24, 16)
    topk = 96
    idx = torch.full((8, topk), -1, dtype=torch.int64)
    counts = [0, 1, 17, 63, 64, 65, 80, 96]
    for r, c in enumerate(counts):
        idx[r, :c] = torch.randint(0, 40, (c,), generator=gen)
    holes = torch.rand(8, topk, generator=gen) < 0.2
    holes[:, 0] = False
    idx = torch.where(holes & (idx >= 0), torch.full_like(idx, -1), idx)
    fixed = idx.to(torch.int32).view(8, 1, topk)
    base = oracle.sparse_mla_fwd(q, kv, fixed, 0.2, 16, lib=lib)
    derived = base[3]
    same = oracle.sparse_mla_fwd(q, kv, fixed, 0.2, 16, topk_length=torch.tensor(derived), lib=lib)
    for a, b in zip(base, same):
        assert np.array_equal(a, b), "derived vs explicit length"
    lens = torch.tensor(counts, dtype=torch.int32)
    dyn = idx.clone()
    for r, c in enumerate(counts):
        dyn[r, c:] = INT32_MAX
    dyn_out = oracle.sparse_mla_fwd(q, kv, dyn.to(torch.int32).view(8, 1, topk), 0.2, 16,
                                    topk_length=lens, lib=lib)
    for a, b in zip(base[:3], dyn_out[:3]):
        assert np.array_equal(a, b), "fixed vs dynamic"
    for enc in (-2, -(2**31), 40, 41, INT32_MAX):
        alt = torch.where(idx < 0, torch.full_like(idx, enc), idx)
        alt_out = oracle.sparse_mla_fwd(q, kv, alt.to(torch.int32).view(8, 1, topk), 0.2, 16, lib=lib)
        for a, b in zip(base, alt_out):
            assert np.array_equal(a, b), f"invalid encoding {enc}"


def pin_nan_in_unreferenced_rows(lib):
    """KV rows that no valid position names may hold NaN without effect, and
    neither may rows named only at positions past an explicit length."""
    gen, q, kv = _tiny(61, 5, 30, 2, 16, 16)
    idx = torch.full((5, 1, 20), -1, dtype=torch.int32)
    for r in range(5):
        idx[r, 0, :10] = torch.randperm(15, generator=gen)[:10].to(torch.int32)
        idx[r, 0, 12] = 20 + r  # named past the explicit length below
    tl = torch.full((5,), 10, dtype=torch.int32)
    clean = oracle.sparse_mla_fwd(q, kv, idx, 0.3, 16, topk_length=tl, lib=lib)
    poisoned = kv.clone()
    poisoned[15:] = float("nan")
    dirty = oracle.sparse_mla_fwd(q, poisoned, idx, 0.3, 16, topk_length=tl, lib=lib)
    for a, b in zip(clean, dirty):
        assert np.array_equal(a, b), "NaN leaked"


def _tiny_decode(seed, B=3, s_q=2, h_q=3, d_qk=24, d_v=16, topk=50, page=8):
    gen = torch.Generator().manual_seed(seed)
    seqlens = torch.tensor([37, 8, 60][:B], dtype=torch.int32)
    npages = [(int(s) + page - 1) // page for s in seqlens]
    mbps = max(npages) + 1
    num_blocks = sum(npages) + 4
    q = _bf16((B, s_q, h_q, d_qk), gen)
    cache = _bf16((num_blocks, page, 1, d_qk), gen)
    perm = torch.randperm(num_blocks, generator=gen)
    bt = torch.full((B, mbps), -1, dtype=torch.int32)
    cur = 0
    for b in range(B):
        bt[b, :npages[b]] = perm[cur:cur + npages[b]].to(torch.int32)
        cur += npages[b]
    cache[perm[cur:]] = float("nan")
    for b in range(B):
        tail = int(seqlens[b]) - (npages[b] - 1) * page
        cache[int(bt[b, npages[b] - 1]), tail:] = float("nan")
    idx = torch.randint(-2, 70, (B, s_q, topk), generator=gen)
    idx[0, 1, 30:] = INT32_MAX
    return q, cache, bt, seqlens, idx.to(torch.int32), gen


def pin_decode_equals_gathered_prefill(lib):
    """Paged decode equals the multiplicity brute force run on each request's
    KV gathered into a contiguous tensor with numpy indexing."""
    page = 8
    q, cache, bt, seqlens, idx, gen = _tiny_decode(71, page=page)
    B, s_q, h_q, d_qk = q.shape
    d_v = 16
    sink = torch.randn(h_q, generator=gen)
    for tl in (None, torch.randint(0, 55, (B, s_q), generator=gen).to(torch.int32)):
        out, lse, ml, rl = oracle.sparse_mla_decode_fwd(q, cache, bt, seqlens, idx, 0.17, d_v,
                                                        attn_sink=sink, topk_length=tl, lib=lib)
        for b in range(B):
            n = int(seqlens[b])
            pos = np.arange(n)
            phys = bt[b].numpy()[pos // page] * page + pos % page
            contig = cache.view(-1, 1, d_qk)[torch.from_numpy(phys)]
            ro, rls, rml, rlen = _multiplicity_reference(
                q[b], contig, idx[b].view(s_q, 1, -1), 0.17, d_v,
                topk_length=None if tl is None else tl[b], sink=sink)
            sl = slice(b * s_q, (b + 1) * s_q)
            assert np.array_equal(rl[sl], rlen)
            _close(out[sl], ro, rtol=1e-10, atol=1e-12, what="decode out")
            _close(lse[sl], rls, what="decode lse")
            _close(ml[sl], rml, what="decode max_logits")
            assert np.all(np.isfinite(out[sl]))
    # a cache length beyond what the block table can address is cut to it
    mbps = bt.shape[1]
    over = seqlens.clone()
    over[0] = mbps * page + 9
    idx2 = idx.clone()
    idx2[0, 0, :12] = torch.arange(mbps * page - 2, mbps * page + 10, dtype=torch.int32)
    idx2[0, 0, 12:] = -1
    ref = oracle.sparse_mla_decode_fwd(q, cache, bt, seqlens, idx2, 0.17, d_v, lib=lib)
    ref_len = oracle.row_lengths(idx2, None, seqlens, rows_per_seq=s_q, addressable=mbps * page,
                                 lib=lib)
    long = oracle.sparse_mla_decode_fwd(q, cache, bt, over, idx2, 0.17, d_v, lib=lib)
    long_len = oracle.row_lengths(idx2, None, over, rows_per_seq=s_q, addressable=mbps * page,
                                  lib=lib)
    # row 0 keeps only the two positions below the addressable limit
    assert long_len[0] == 2 and long[3][0] == 2
    for r in range(s_q, B * s_q):  # other requests are untouched
        assert np.array_equal(long[0][r], ref[0][r]) and long_len[r] == ref_len[r]


def pin_decode_page_range_mask(lib):
    """A valid position whose block-table entry lies outside [0, num_blocks)
    is masked like an invalid index (reading of FlashMLA PR #216,
    "Correctness": no illegal memory access), while the tail scan still reads
    index values only.  Every other key is kept, among them keys on physical
    pages 0 and num_blocks - 1 and on a page two requests share.  Checked on
    every row, with and without explicit lengths and with a sink, against
    the numpy multiplicity brute force over the request's keys with those
    positions dropped."""
    page, num_blocks = 8, 9
    gen = torch.Generator().manual_seed(97)
    B, s_q, h_q, d_qk, d_v, topk = 2, 3, 3, 24, 16, 40
    seqlens = torch.tensor([48, 40], dtype=torch.int32)
    # logical pages: request 0 -> 0, -1, 8, num_blocks, 3, 5; request 1 ->
    # num_blocks + 3, 7, 1, -7, 8 (physical page 8 is shared)
    bt = torch.tensor([[0, -1, 8, num_blocks, 3, 5, 2],
                       [num_blocks + 3, 7, 1, -7, 8, 4, 6]], dtype=torch.int32)
    q = _bf16((B, s_q, h_q, d_qk), gen)
    cache = _bf16((num_blocks, page, 1, d_qk), gen)
    sink = torch.randn(h_q, generator=gen)
    idx = torch.full((B, s_q, topk), -1, dtype=torch.int32)
    for b in range(B):
        n = int(seqlens[b])
        for t in range(s_q):
            k = 30 - 4 * t
            idx[b, t, :k] = torch.randperm(n, generator=gen)[:k].to(torch.int32)
    # the last valid entry of these rows sits on a masked page: the derived
    # length still counts it (the tail scan reads index values only)
    idx[0, 0, 29] = 1 * page + 3      # logical page 1 -> -1
    idx[1, 1, 25] = 0 * page + 5      # logical page 0 -> num_blocks + 3
    idx[0, 2, 33] = 3 * page + 1      # logical page 3 -> num_blocks, past -1 padding
    # every position of this row is on a masked page: the row has no key
    idx[1, 2, :6] = torch.tensor([3, 30, 25, 1, 26, 7], dtype=torch.int32)
    idx[1, 2, 6:] = -1
    cache_v = cache.view(-1, 1, d_qk)
    bt_n = bt.numpy().astype(np.int64)
    for tl in (None, torch.tensor([[40, 12, 34], [3, 26, 6]], dtype=torch.int32)):
        out, lse, ml, rl = oracle.sparse_mla_decode_fwd(q, cache, bt, seqlens, idx, 0.21, d_v,
                                                        attn_sink=sink, topk_length=tl, lib=lib)
        for b in range(B):
            n = int(seqlens[b])
            pos = np.arange(n)
            pg = bt_n[b][pos // page]
            on_pool = (pg >= 0) & (pg < num_blocks)
            phys = np.where(on_pool, pg, 0) * page + pos % page
            contig = cache_v[torch.from_numpy(phys)]
            ib = idx[b].numpy().astype(np.int64)
            in_range = (ib >= 0) & (ib < n)
            kept = in_range & on_pool[np.where(in_range, ib, 0)]
            # lengths: the index values against the cache length alone
            if tl is None:
                want_len = np.array([(np.nonzero(r)[0][-1] + 1) if r.any() else 0
                                     for r in in_range])
            else:
                want_len = np.clip(tl[b].numpy(), 0, topk)
            dropped = torch.from_numpy(np.where(kept, ib, -1).astype(np.int32))
            ro, rls, rml, _ = _multiplicity_reference(
                q[b], contig, dropped.view(s_q, 1, -1), 0.21, d_v,
                topk_length=torch.from_numpy(want_len.astype(np.int32)), sink=sink)
            sl = slice(b * s_q, (b + 1) * s_q)
            assert np.array_equal(rl[sl], want_len), "decode row length"
            _close(out[sl], ro, rtol=1e-10, atol=1e-12, what="decode page-range out")
            _close(lse[sl], rls, what="decode page-range lse")
            _close(ml[sl], rml, what="decode page-range max_logits")
        # the row whose keys are all on masked pages gives the empty-row triple
        assert np.all(out[5] == 0) and np.all(lse[5] == np.inf) and np.all(ml[5] == -np.inf)


def pin_row_selection(lib):
    """Evaluating a subset of rows returns exactly those rows of the full run."""
    gen, q, kv = _tiny(81, 7, 30, 2, 16, 16)
    idx = torch.randint(-2, 33, (7, 1, 25), generator=gen).to(torch.int32)
    full = oracle.sparse_mla_fwd(q, kv, idx, 0.3, 16, lib=lib)
    sel = np.array([6, 0, 3])
    part = oracle.sparse_mla_fwd(q, kv, idx, 0.3, 16, rows=sel, lib=lib)
    for a, b in zip(full, part):
        assert np.array_equal(a[sel], b)


# ---------------------------------------------------------------------------
# backward pins
# ---------------------------------------------------------------------------

def _dense_bwd_reference(q, kv, indices, sm_scale, d_v, dout, topk_length=None, sink=None):
    """float64 torch autograd of dense attention over every KV row with bias
    ln(count) (count: how often a row is named before the row's length) and,
    with a sink, one more value-less column of logit sink[h].  Returns
    (out, sink-free lse, dq, dkv, d_sink); rows without keys are left out of
    the loss (out 0, lse +inf)."""
    qd = _f64(q).clone().requires_grad_(True)
    kvd = _f64(kv[:, 0, :]).clone().requires_grad_(True)
    sd = None if sink is None else sink.to(torch.float64).clone().requires_grad_(True)
    idx = indices.reshape(indices.shape[0], -1).numpy().astype(np.int64)
    s_q, h_q, _ = qd.shape
    s_kv = kvd.shape[0]
    topk = idx.shape[1]
    out = torch.zeros(s_q, h_q, d_v, dtype=torch.float64)
    lse = torch.full((s_q, h_q), math.inf, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for r in range(s_q):
        valid = (idx[r] >= 0) & (idx[r] < s_kv)
        if topk_length is None:
            nz = np.nonzero(valid)[0]
            L = int(nz[-1]) + 1 if nz.size else 0
        else:
            L = int(min(max(int(topk_length[r]), 0), topk))
        count = np.bincount(idx[r, :L][valid[:L]], minlength=s_kv).astype(np.float64)
        if count.sum() == 0:
            continue
        with np.errstate(divide="ignore"):
            bias = torch.from_numpy(np.log(count))
        scores = sm_scale * (qd[r] @ kvd.T) + bias[None, :]
        full = scores if sd is None else torch.cat([scores, sd[:, None]], dim=1)
        p = torch.softmax(full, dim=1)[:, :s_kv]
        o = p @ kvd[:, :d_v]
        loss = loss + (_f64(dout[r]) * o).sum()
        out[r] = o.detach()
        lse[r] = torch.logsumexp(scores, dim=1).detach()
    loss.backward()
    d_sink = None if sd is None else sd.grad.numpy()
    return out, lse, qd.grad.numpy(), kvd.grad.numpy(), d_sink


def _bwd_case(seed, s_q=6, s_kv=29, h_q=3, d_qk=20, d_v=12, topk=17):
    gen, q, kv = _tiny(seed, s_q, s_kv, h_q, d_qk, d_v)
    idx = torch.randint(0, s_kv, (s_q, 1, topk), generator=gen).to(torch.int32)
    idx[0, 0, 3] = idx[0, 0, 1]            # a repeated key
    idx[1, 0, -4:] = -1                    # -1 padded tail
    idx[2, 0, 5] = s_kv                    # invalid entries inside the row
    idx[2, 0, 7] = INT32_MAX
    idx[3, 0, :] = -1                      # a row without keys
    dout = _bf16((s_q, h_q, d_v), gen)
    return gen, q, kv, idx, dout


def pin_bwd_equals_autograd(lib):
    """dq, dkv (and d_sink) equal float64 autograd of the dense formulation,
    with and without topk_length and a sink."""
    for seed, with_len, with_sink in [(201, False, False), (202, True, False), (203, False, True),
                                      (204, True, True)]:
        gen, q, kv, idx, dout = _bwd_case(seed)
        s_q, h_q = q.shape[0], q.shape[1]
        tl = torch.randint(0, idx.shape[-1] + 3, (s_q,), generator=gen).to(torch.int32) \
            if with_len else None
        sink = (torch.randn(h_q, generator=gen) * 2).to(torch.float32) if with_sink else None
        scale = 0.45
        out, lse, dq_ref, dkv_ref, ds_ref = _dense_bwd_reference(q, kv, idx, scale, 12, dout, tl,
                                                                 sink)
        dq, dkv, ds = oracle.sparse_mla_bwd(q, kv, out, dout, idx, lse, scale, 12, attn_sink=sink,
                                            topk_length=tl, want_d_sink=with_sink, lib=lib)
        _close(dq, dq_ref, 1e-9, 1e-11, f"dq seed {seed}")
        _close(dkv, dkv_ref, 1e-9, 1e-11, f"dkv seed {seed}")
        if with_sink:
            _close(ds, ds_ref, 1e-9, 1e-11, f"d_sink seed {seed}")
        assert np.all(dq[3] == 0.0), "a row without keys has a zero dq"


def pin_bwd_single_key(lib):
    """One key per row: out = v and p = 1, so dq = 0 and the key's row gets the
    sum of dout over its heads (and rows) in the value columns, nothing else."""
    gen, q, kv = _tiny(211, 5, 11, 3, 20, 12)
    keys = torch.tensor([4, 7, 4, 0, 10], dtype=torch.int32)
    idx = torch.full((5, 1, 6), -1, dtype=torch.int32)
    idx[torch.arange(5), 0, torch.tensor([0, 2, 5, 1, 3])] = keys
    dout = _bf16((5, 3, 12), gen)
    kvn = _f64(kv[:, 0, :]).numpy()
    out = np.stack([np.tile(kvn[int(k), :12], (3, 1)) for k in keys])
    lse = np.stack([0.3 * (_f64(q[r]).numpy() @ kvn[int(keys[r])]) for r in range(5)])
    dq, dkv, _ = oracle.sparse_mla_bwd(q, kv, out, dout, idx, lse, 0.3, 12, lib=lib)
    assert np.abs(dq).max() < 1e-12, "dq of single-key rows"
    want = np.zeros((11, 20))
    for r in range(5):
        want[int(keys[r]), :12] += _f64(dout[r]).numpy().sum(axis=0)
    _close(dkv, want, 1e-12, 1e-12, "dkv of single-key rows")


def pin_bwd_base2_and_selection(lib):
    """Base-2 lse gives the natural-log result; row and KV-row selections are
    exactly the matching slices of the full result."""
    gen, q, kv, idx, dout = _bwd_case(221)
    out, lse, *_ = _dense_bwd_reference(q, kv, idx, 0.45, 12, dout)
    dq, dkv, _ = oracle.sparse_mla_bwd(q, kv, out, dout, idx, lse, 0.45, 12, lib=lib)
    dq2, dkv2, _ = oracle.sparse_mla_bwd(q, kv, out, dout, idx, lse / math.log(2), 0.45, 12,
                                         lse_base2=True, lib=lib)
    _close(dq2, dq, 1e-12, 1e-14, "dq, base-2 lse")
    _close(dkv2, dkv, 1e-12, 1e-14, "dkv, base-2 lse")
    rows, krows = np.array([5, 0, 2]), np.array([28, 3, 3, 11])
    dq3, dkv3, _ = oracle.sparse_mla_bwd(q, kv, out, dout, idx, lse, 0.45, 12, rows=rows,
                                         kv_rows=krows, lib=lib)
    assert np.array_equal(dq3, dq[rows]) and np.array_equal(dkv3, dkv[krows])



# ---------------------------------------------------------------------------
# block-sparse forward pins
# ---------------------------------------------------------------------------

def _bs_tiny(seed, s=45, h_q=4, h_kv=2, d_qk=24, d_v=16):
    gen = torch.Generator().manual_seed(seed)
    return gen, _bf16((s, h_q, d_qk), gen), _bf16((s, h_kv, d_qk), gen), _bf16((s, h_kv, d_v), gen)


def _csr(lists):
    ptr = np.zeros(len(lists) + 1, dtype=np.int32)
    ptr[1:] = np.cumsum([len(x) for x in lists])
    col = np.array([b for x in lists for b in x], dtype=np.int32)
    return torch.from_numpy(ptr), torch.from_numpy(col)


def _sdpa(q, k, v, scale, causal):
    """torch SDPA in float64 with grouped KV heads; returns (out, lse)."""
    qd, kd, vd = (_f64(x).permute(1, 0, 2) for x in (q, k, v))
    g = qd.shape[0] // kd.shape[0]
    kd, vd = kd.repeat_interleave(g, 0), vd.repeat_interleave(g, 0)
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, scale=scale, is_causal=causal)
    sc = scale * (qd @ kd.transpose(1, 2))
    if causal:
        n = sc.shape[-1]
        sc = sc.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -math.inf)
    return out.permute(1, 0, 2).numpy(), torch.logsumexp(sc, -1).T.numpy()


def pin_block_sparse_full_selection_is_dense(lib):
    """Selecting every key block up to the diagonal (causal), or every block
    (not causal), is dense attention."""
    for seed, (q_block, k_block) in [(301, (8, 4)), (302, (16, 16)), (303, (6, 10))]:
        gen, q, k, v = _bs_tiny(seed)
        s = q.shape[0]
        nq, nk = -(-s // q_block), -(-s // k_block)
        scale = 0.6 / math.sqrt(q.shape[2])
        causal_lists = [list(range(min(nk, ((qb + 1) * q_block - 1) // k_block + 1)))[::-1]
                        for qb in range(nq)]
        for causal, lists in [(True, causal_lists), (False, [list(range(nk))] * nq)]:
            ptr, col = _csr(lists)
            out, lse = oracle.block_sparse_fwd(q, k, v, ptr, col, q_block, k_block, scale,
                                               causal=causal, lib=lib)
            ref_out, ref_lse = _sdpa(q, k, v, scale, causal)
            _close(out, ref_out, 1e-11, 1e-12, f"block-sparse out (causal={causal})")
            _close(lse, ref_lse, 1e-11, 1e-12, f"block-sparse lse (causal={causal})")


def pin_block_sparse_bruteforce(lib):
    """Random selections (repeated and out-of-range block ids, empty lists)
    against dense attention with bias ln(count) over a numpy mask."""
    for seed, causal in [(311, True), (312, False)]:
        gen, q, k, v = _bs_tiny(seed, s=37, h_q=6, h_kv=3)
        s, h_q, _ = q.shape
        q_block, k_block = 8, 6
        nq, nk = -(-s // q_block), -(-s // k_block)
        lists = []
        for qb in range(nq):
            n = int(torch.randint(0, nk + 2, (1,), generator=gen))
            lists.append([int(b) for b in torch.randint(-1, nk + 2, (n,), generator=gen)])
        lists[0] = []
        lists[1] = [2, 2, 0]
        ptr, col = _csr(lists)
        out, lse = oracle.block_sparse_fwd(q, k, v, ptr, col, q_block, k_block, 0.4, causal=causal,
                                           lib=lib)
        qn, kn, vn = _f64(q).numpy(), _f64(k).numpy(), _f64(v).numpy()
        g = h_q // kn.shape[1]
        for i in range(s):
            count = np.zeros(s)
            for b in lists[i // q_block]:
                if 0 <= b < nk:
                    count[b * k_block:min((b + 1) * k_block, s)] += 1
            if causal:
                count[i + 1:] = 0
            for h in range(h_q):
                if count.sum() == 0:
                    assert np.all(out[i, h] == 0) and lse[i, h] == math.inf, "empty row"
                    continue
                with np.errstate(divide="ignore"):
                    sc = 0.4 * (kn[:, h // g] @ qn[i, h]) + np.log(count)
                m = sc.max()
                w = np.exp(sc - m)
                _close(out[i, h], (w @ vn[:, h // g]) / w.sum(), 1e-11, 1e-12, f"row {i} head {h}")
                _close(lse[i, h], m + np.log(w.sum()), 1e-11, 1e-12, f"lse row {i} head {h}")


ALL_PINS = [
    pin_dense_equals_library_attention,
    pin_sink_equals_extra_key,
    pin_sink_closed_form,
    pin_multiplicity_bruteforce,
    pin_closed_forms,
    pin_empty_rows,
    pin_row_length_fixtures,
    pin_row_length_bruteforce,
    pin_length_and_encoding_invariance,
    pin_nan_in_unreferenced_rows,
    pin_decode_equals_gathered_prefill,
    pin_decode_page_range_mask,
    pin_row_selection,
    pin_bwd_equals_autograd,
    pin_bwd_single_key,
    pin_bwd_base2_and_selection,
    pin_block_sparse_full_selection_is_dense,
    pin_block_sparse_bruteforce,
]
