"""Seeded synthetic inputs for sparse top-k MLA attention (prefill and paged decode).

This module only draws inputs: query/KV payloads, index vectors, optional
per-row lengths, attention sinks, block tables and sequence lengths.  It holds
none of the attention arithmetic, so both the HIP path and the CPU oracle can
take their inputs from it.

Shapes and structure follow the workloads measured on the pages:
  * FlashMLA PR #196, "Numbers": bf16 prefill with s_q = 8192, h_q = 64,
    h_kv = 1, d_qk = d_v = 512, rows front-packed with causal indices whose
    count ramps up to ~1027 and padded with -1 to a width of 1152.
  * FlashMLA PR #196, "Correctness notes": scattered interior invalids (-1 and
    >= s_kv mid-row), all-invalid rows, head128 with topk 2048 at d_qk 576,
    with and without attn_sink.
  * FlashMLA PR #216, "Dynamic top-k": B = 256, S_q = 1, H = 128, d_qk = 576,
    s_kv = 4096, 64-token pages, allocated top-k 2048, effective length 1024,
    suffix poisoned with INT_MAX.
  * FlashMLA PR #216, "Fixed top-k regression check": S_q = 2, H = 128,
    d_qk = 576, variable KV lengths up to 32768, page block 64, topk = 2048.

Every tensor is produced on the CPU from one ``torch.Generator`` per case, in
a fixed draw order (q, kv, indices, sink, lengths / block table), so a seed
fully determines a case.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

INT32_MAX = 2**31 - 1
PAGE_SIZE = 64


@dataclass
class PrefillCase:
    name: str
    q: torch.Tensor  # bf16 [s_q, h_q, d_qk]
    kv: torch.Tensor  # bf16 [s_kv, 1, d_qk]; V is kv[..., :d_v]
    indices: torch.Tensor  # int32 [s_q, 1, topk]
    topk_length: Optional[torch.Tensor]  # int32 [s_q] or None
    attn_sink: Optional[torch.Tensor]  # fp32 [h_q] or None
    sm_scale: float
    d_v: int
    meta: dict = field(default_factory=dict)

    @property
    def s_q(self):
        return self.q.shape[0]

    @property
    def h_q(self):
        return self.q.shape[1]

    @property
    def d_qk(self):
        return self.q.shape[2]

    @property
    def s_kv(self):
        return self.kv.shape[0]

    @property
    def topk(self):
        return self.indices.shape[-1]


@dataclass
class DecodeCase:
    name: str
    q: torch.Tensor  # bf16 [B, s_q, h_q, d_qk]
    kv_cache: torch.Tensor  # bf16 [num_blocks, page_size, 1, d_qk]
    block_table: torch.Tensor  # int32 [B, max_blocks_per_seq]
    cache_seqlens: torch.Tensor  # int32 [B]
    indices: torch.Tensor  # int32 [B, s_q, topk] logical token positions
    topk_length: Optional[torch.Tensor]  # int32 [B, s_q] or None
    attn_sink: Optional[torch.Tensor]  # fp32 [h_q] or None
    sm_scale: float
    d_v: int
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def s_q(self):
        return self.q.shape[1]

    @property
    def h_q(self):
        return self.q.shape[2]

    @property
    def d_qk(self):
        return self.q.shape[3]

    @property
    def topk(self):
        return self.indices.shape[-1]

    @property
    def page_size(self):
        return self.kv_cache.shape[1]


def _as_f32(x):
    """The softmax scale crosses the C boundary as a binary32; keep the case's
    value at exactly that precision so every consumer sees the same number."""
    return float(torch.tensor(x, dtype=torch.float32).item())


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------

def _randn_bf16(shape, gen, chunk_elems=1 << 26):
    """N(0,1) fp32 draws rounded to bf16, produced in chunks to bound memory."""
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        stop = min(n, start + chunk_elems)
        flat[start:stop] = torch.randn(stop - start, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    return out


def _random_subsets(rows, universe, take, gen, upper=None, count=None):
    """For each row r, the first entries of a uniformly random ordering of
    [0, upper[r]) (or of [0, universe) when `upper` is None).  A row keeps
    `count[r]` of them (default: all that fit in `take`); the positions after
    those hold -1.  Returns int64 [rows, take]."""
    keys = torch.rand(rows, universe, generator=gen)
    col = torch.arange(universe).unsqueeze(0)
    if upper is not None:
        keys = torch.where(col < upper.unsqueeze(1), keys, torch.full_like(keys, 2.0))
    order = torch.argsort(keys, dim=1)[:, :take]
    keep = upper if count is None else (count if upper is None else torch.minimum(count, upper))
    if keep is not None:
        pos = torch.arange(order.shape[1]).unsqueeze(0)
        order = torch.where(pos < keep.unsqueeze(1), order, torch.full_like(order, -1))
    return order


def _invalid_values(n, s_kv, gen):
    """Invalid index encodings: -1, other negatives, exactly s_kv, INT32_MAX and
    values in (s_kv, 2*s_kv)."""
    u = torch.rand(n, generator=gen)
    big = torch.randint(s_kv + 1, 2 * s_kv, (n,), generator=gen)
    neg = -torch.randint(2, 1000, (n,), generator=gen)
    vals = torch.full((n,), -1, dtype=torch.int64)
    vals = torch.where((u >= 0.45) & (u < 0.5), neg, vals)
    vals = torch.where((u >= 0.5) & (u < 0.6), torch.full_like(vals, s_kv), vals)
    vals = torch.where((u >= 0.6) & (u < 0.7), torch.full_like(vals, INT32_MAX), vals)
    vals = torch.where(u >= 0.7, big, vals)
    return vals


# ---------------------------------------------------------------------------
# prefill cases
# ---------------------------------------------------------------------------

def make_prefill(name, *, s_q, s_kv, h_q, d_qk, d_v, topk, layout, seed,
                 ramp_cap=None, invalid_frac=0.0, empty_frac=0.0,
                 with_length=False, with_sink=False, sm_scale=None, row_offset=0):
    """Generic prefill case.

    layout:
      "ramp"      row i (absolute row i + row_offset) holds min(i+1, ramp_cap)
                  distinct keys drawn from the causal range [0, i] in random
                  order, front-packed, then -1 padding up to `topk`.
      "scattered" every row holds `topk` distinct keys from [0, s_kv) in random
                  order; each position independently becomes an invalid value
                  with probability `invalid_frac`; a fraction `empty_frac` of
                  the rows is made entirely invalid.
      "full"      every row holds `topk` distinct keys from [0, s_kv), all valid.
    """
    gen = torch.Generator().manual_seed(seed)
    q = _randn_bf16((s_q, h_q, d_qk), gen)
    kv = _randn_bf16((s_kv, 1, d_qk), gen)
    meta = {"layout": layout}
    if layout == "ramp":
        cap = topk if ramp_cap is None else ramp_cap
        absrow = torch.arange(s_q) + row_offset
        upper = torch.clamp(absrow + 1, max=s_kv)
        counts = torch.clamp(upper, max=cap)
        universe = int(upper.max().item())
        idx = _random_subsets(s_q, universe, min(topk, universe), gen, upper=upper, count=counts)
        if idx.shape[1] < topk:
            idx = torch.cat([idx, torch.full((s_q, topk - idx.shape[1]), -1, dtype=idx.dtype)], dim=1)
        lengths = counts.to(torch.int32)
        meta["ramp_cap"] = cap
    elif layout in ("scattered", "full"):
        idx = _random_subsets(s_q, s_kv, topk, gen)
        lengths = None
        if layout == "scattered":
            inval = torch.rand(s_q, topk, generator=gen) < invalid_frac
            vals = _invalid_values(int(inval.sum().item()), s_kv, gen)
            idx[inval] = vals
            n_empty = int(round(empty_frac * s_q))
            if n_empty:
                rows = torch.randperm(s_q, generator=gen)[:n_empty]
                idx[rows] = _invalid_values(n_empty * topk, s_kv, gen).view(n_empty, topk)
                meta["empty_rows"] = sorted(rows.tolist())
        else:
            lengths = torch.full((s_q,), topk, dtype=torch.int32)
    else:
        raise ValueError(layout)
    indices = idx.to(torch.int32).view(s_q, 1, topk).contiguous()
    sink = torch.randn(h_q, generator=gen, dtype=torch.float32) if with_sink else None
    topk_length = None
    if with_length:
        if lengths is None:
            raise ValueError("layout has no natural per-row length")
        topk_length = lengths.contiguous()
    scale = _as_f32((1.0 / math.sqrt(d_qk)) if sm_scale is None else sm_scale)
    return PrefillCase(name, q, kv, indices, topk_length, sink, scale, d_v, meta)


def tiny_prefill(seed=0):
    """s_q=64, s_kv=256, h_q=16, d_qk=576, d_v=512, topk=64; row i holds all of
    [0, i] in random order, then -1; no length, no sink; sm_scale=1/sqrt(576)."""
    return make_prefill("tiny_prefill_h16_d576", s_q=64, s_kv=256, h_q=16, d_qk=576, d_v=512,
                        topk=64, layout="ramp", seed=seed)


def prefill_h64(with_length=False, seed=0, s_q=8192, s_kv=8192, row_offset=0):
    """s_q=s_kv=8192, h_q=64, d_qk=d_v=512, width 1152, row i holds
    min(i+1, 1027) distinct causal keys then -1 (ramp-padded)."""
    tag = "len" if with_length else "nolen"
    return make_prefill(f"prefill_h64_d512_ramp1027_w1152_{tag}", s_q=s_q, s_kv=s_kv, h_q=64,
                        d_qk=512, d_v=512, topk=1152, layout="ramp", ramp_cap=1027, seed=seed,
                        with_length=with_length, row_offset=row_offset)


def prefill_h128(seed=0, s_q=4096, s_kv=4096, topk=2048):
    """s_q=s_kv=4096, h_q=128, d_qk=576, d_v=512, topk=2048, ~10% scattered
    invalids, 1% all-invalid rows, per-head fp32 sink."""
    return make_prefill("prefill_h128_d576_scatter10_sink", s_q=s_q, s_kv=s_kv, h_q=128, d_qk=576,
                        d_v=512, topk=topk, layout="scattered", invalid_frac=0.10,
                        empty_frac=0.01, with_sink=True, seed=seed)


def bwd_h64(seed=0, s_q=4096, s_kv=4096, topk=2048, d_qk=576):
    """Backward shape of the pages: T = s_q = s_kv = 4096, h_q = 64,
    d_qk = 576, d_v = 512, topk = 2048; row i holds min(i + 1, 2048) distinct
    causal keys in random order, then -1 (causal top-k selection)."""
    return make_prefill(f"bwd_h64_d{d_qk}_T{s_q}_topk{topk}", s_q=s_q, s_kv=s_kv, h_q=64,
                        d_qk=d_qk, d_v=512, topk=topk, layout="ramp", ramp_cap=topk, seed=seed,
                        with_length=True)


def bwd_dout(case, seed):
    """Seeded gradient of the forward output: bf16 [s_q, h_q, d_v], N(0, 1)."""
    gen = torch.Generator().manual_seed(seed)
    return _randn_bf16((case.s_q, case.h_q, case.d_v), gen)


def bwd_synthetic_stats(case, seed):
    """Seeded stand-ins for the forward's out and lse when the forward itself
    is too costly to evaluate on the CPU: lse = ln(keys of the row) + 1/2 + a
    little noise (the size of the normaliser for unit-variance logits), out =
    N(0, 1) / sqrt(keys), bf16 (the size of a softmax average of unit values).
    Rows without keys get lse = +inf and out = 0."""
    gen = torch.Generator().manual_seed(seed)
    lens = case.topk_length.to(torch.float64) if case.topk_length is not None else None
    if lens is None:
        raise ValueError("case needs explicit row lengths")
    n = torch.clamp(lens, min=1.0)
    lse = (torch.log(n) + 0.5)[:, None] + 0.1 * torch.randn(case.s_q, case.h_q, generator=gen,
                                                              dtype=torch.float64)
    lse = torch.where((lens > 0)[:, None], lse, torch.full_like(lse, math.inf))
    out = _randn_bf16((case.s_q, case.h_q, case.d_v), gen).to(torch.float32)
    out = (out / torch.sqrt(n).to(torch.float32)[:, None, None]) * (lens > 0).to(torch.float32)[:, None, None]
    return out.to(torch.bfloat16), lse.to(torch.float32)


@dataclass
class BlockSparseCase:
    name: str
    q: torch.Tensor            # [s, h_q, 192] bf16
    k: torch.Tensor            # [s, h_kv, 192] bf16
    v: torch.Tensor            # [s, h_kv, 128] bf16
    row_ptr: torch.Tensor      # [ceil(s / q_block) + 1] int32
    col_idx: torch.Tensor      # [nnz] int32
    q_block: int
    k_block: int
    causal: bool
    sm_scale: float

    @property
    def s(self):
        return self.q.shape[0]

    @property
    def h_q(self):
        return self.q.shape[1]


def _csr(lists):
    ptr = torch.zeros(len(lists) + 1, dtype=torch.int32)
    ptr[1:] = torch.cumsum(torch.tensor([len(x) for x in lists], dtype=torch.int64), 0).to(torch.int32)
    col = torch.tensor([b for x in lists for b in x], dtype=torch.int32)
    return ptr, col


def make_block_sparse(name, *, s, h_q, h_kv, q_block, k_block, selection, seed, causal=True,
                      window=4, density=0.3):
    """Block-sparse case (192/128 heads).  selection:
      "sink_window"  key block 0 plus the `window` key blocks that end at the
                     query block's last row (the pages' benchmark selection)
      "full_causal"  every key block up to that one (dense causal attention)
      "random"       each key block up to that one with probability
                     `density`, in random order, plus a few ids out of range"""
    gen = torch.Generator().manual_seed(seed)
    q = _randn_bf16((s, h_q, 192), gen)
    k = _randn_bf16((s, h_kv, 192), gen)
    v = _randn_bf16((s, h_kv, 128), gen)
    nq, nk = -(-s // q_block), -(-s // k_block)
    lists = []
    for qb in range(nq):
        last = min(nk - 1, (min((qb + 1) * q_block, s) - 1) // k_block) if causal else nk - 1
        if selection == "sink_window":
            sel = list(range(max(0, last - window + 1), last + 1))
            if 0 not in sel:
                sel = [0] + sel
        elif selection == "full_causal":
            sel = list(range(last + 1))
        elif selection == "random":
            keep = torch.rand(last + 1, generator=gen) < density
            sel = [int(b) for b in torch.nonzero(keep).flatten()]
            sel = [sel[i] for i in torch.randperm(len(sel), generator=gen).tolist()]
            if torch.rand(1, generator=gen).item() < 0.3:
                sel.append(int(nk + torch.randint(0, 3, (1,), generator=gen)))
                sel.append(-1)
        else:
            raise ValueError(selection)
        lists.append(sel)
    ptr, col = _csr(lists)
    return BlockSparseCase(name, q, k, v, ptr, col, q_block, k_block, causal,
                           _as_f32(1.0 / math.sqrt(192)))


def block_sparse_h8(seed=0, s=65536):
    """The pages' block-sparse forward benchmark: h = 8, 192/128 heads,
    q_block 256, k_block 128, causal, key block 0 plus a 4-block window."""
    return make_block_sparse(f"block_sparse_h8_s{s}_sink_window4", s=s, h_q=8, h_kv=8, q_block=256,
                             k_block=128, selection="sink_window", seed=seed)


# ---------------------------------------------------------------------------
# decode cases
# ---------------------------------------------------------------------------

def make_decode(name, *, batch, s_q, h_q, d_qk, d_v, topk, seqlens, seed,
                effective=None, with_length=False, poison=INT32_MAX, with_sink=False,
                spare_pages=1024, max_blocks_per_seq=None, sm_scale=None):
    """Generic paged decode case.

    `seqlens` is an int tensor [batch] of KV lengths.  Each sequence owns
    ceil(len/64) distinct pages of a shared pool, in random positions; the pool
    also holds `spare_pages` pages that no sequence owns.  Spare pages and the
    tokens past a sequence's length in its last page are filled with NaN.

    Each query row (b, t) holds `effective` (default `topk`) distinct logical
    positions from [0, seqlens[b]) in random order; the positions after them
    hold `poison` (INT32_MAX or -1).  With `with_length`, topk_length[b, t] is
    the effective count.
    """
    gen = torch.Generator().manual_seed(seed)
    seqlens = seqlens.to(torch.int64)
    pages_per_seq = (seqlens + PAGE_SIZE - 1) // PAGE_SIZE
    mbps = int(pages_per_seq.max().item()) if max_blocks_per_seq is None else max_blocks_per_seq
    used = int(pages_per_seq.sum().item())
    num_blocks = used + spare_pages

    q = _randn_bf16((batch, s_q, h_q, d_qk), gen)
    kv_cache = _randn_bf16((num_blocks, PAGE_SIZE, 1, d_qk), gen)

    eff = topk if effective is None else effective
    rows = batch * s_q
    upper = seqlens.repeat_interleave(s_q)
    universe = int(seqlens.max().item())
    sub = _random_subsets(rows, universe, min(eff, universe), gen, upper=upper)
    if (upper < eff).any():
        raise ValueError("sequence shorter than the effective top-k")
    idx = torch.full((rows, topk), poison, dtype=torch.int64)
    idx[:, :eff] = sub[:, :eff]
    indices = idx.to(torch.int32).view(batch, s_q, topk).contiguous()

    sink = torch.randn(h_q, generator=gen, dtype=torch.float32) if with_sink else None

    perm = torch.randperm(num_blocks, generator=gen)
    block_table = torch.full((batch, mbps), -1, dtype=torch.int32)
    cursor = 0
    for b in range(batch):
        n = int(pages_per_seq[b].item())
        block_table[b, :n] = perm[cursor:cursor + n].to(torch.int32)
        cursor += n
    spare = perm[cursor:]
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    if spare.numel():
        kv_cache[spare] = nan
    for b in range(batch):
        n = int(pages_per_seq[b].item())
        tail = int(seqlens[b].item()) - (n - 1) * PAGE_SIZE
        if tail < PAGE_SIZE:
            kv_cache[int(block_table[b, n - 1].item()), tail:] = nan

    topk_length = None
    if with_length:
        topk_length = torch.full((batch, s_q), eff, dtype=torch.int32)
    scale = _as_f32((1.0 / math.sqrt(d_qk)) if sm_scale is None else sm_scale)
    meta = {"effective": eff, "spare_pages": spare_pages, "poison": poison}
    return DecodeCase(name, q, kv_cache, block_table, seqlens.to(torch.int32).contiguous(), indices,
                      topk_length, sink, scale, d_v, meta)


def decode_dynamic(with_length=True, seed=0, batch=256):
    """B=256, s_q=1, h_q=128, d_qk=576, seqlen 4096 each, topk 2048 allocated,
    1024 effective, suffix poisoned with INT32_MAX (or -1 without a length)."""
    poison = INT32_MAX if with_length else -1
    tag = "len" if with_length else "nolen"
    return make_decode(f"decode_dyn_b{batch}_h128_d576_k2048_eff1024_{tag}", batch=batch, s_q=1,
                       h_q=128, d_qk=576, d_v=512, topk=2048,
                       seqlens=torch.full((batch,), 4096, dtype=torch.int64), seed=seed,
                       effective=1024, with_length=with_length, poison=poison)


def decode_fixed(seed=0, batch=128, min_len=4096, max_len=32768):
    """B=128, s_q=2, h_q=128, d_qk=576, per-sequence KV length uniform in
    [4096, 32768], topk=2048 distinct valid positions per row, no length."""
    gen = torch.Generator().manual_seed(seed + 7919)
    seqlens = torch.randint(min_len, max_len + 1, (batch,), generator=gen)
    return make_decode(f"decode_fixed_b{batch}_sq2_h128_d576_k2048", batch=batch, s_q=2, h_q=128,
                       d_qk=576, d_v=512, topk=2048, seqlens=seqlens, seed=seed,
                       max_blocks_per_seq=max(512, (max_len + PAGE_SIZE - 1) // PAGE_SIZE))
