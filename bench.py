#!/usr/bin/env python
"""Benchmark of the sparse top-k MLA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the hot path (row lengths, index validity, gather,
S = QK^T, masked online softmax, P.V, finalize) over one batch of synthetic
input that is resident in HBM before timing starts.  The default workload is
the sparse prefill with 64 heads, d_qk = d_v = 512, s_q = s_kv = 8192 and a
1152-wide causal ramp capped at 1027 keys (no topk_length, so the tail scan
runs); the same rows with topk_length are timed beside it.

Prints ONE JSON line: throughput in TFLOP/s over valid (query, key) pairs
(FLOPs = 2 * h_q * (d_qk + d_v) * sum of valid keys, counted from the data),
ms per call, the roofline of the kernel and the CPU oracle timed on a bounded
sample of the same rows.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
PROFILES = ROOT / "profiles"
METRIC = "sparse MLA fwd ms/call + TFLOP/s over valid keys; % MFMA / HBM peak"
METRIC_BWD = "sparse MLA bwd ms/call + TFLOP/s over valid keys; % MFMA peak"
METRIC_BS = "block-sparse MLA fwd ms/call + TFLOP/s over selected (causal) pairs; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_h64",
                    choices=["prefill_h64", "prefill_h64_len", "prefill_h128", "decode_dynamic",
                             "decode_dynamic_nolen", "decode_fixed", "decode_fixed_b2", "tiny",
                             "bwd_h64", "block_sparse_h8"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR (pmc_<workload>_<counter>/ "
                         "and pmc_copy_<counter>/), and the MFMA-busy runs (pmc_<workload>_MFMA/), into "
                         "profiles/traffic_<workload>.json; no GPU needed")
    ap.add_argument("--attainable", action="store_true",
                    help="measure this device's attainable dense bf16 MFMA rate (an MFMA loop), HBM "
                         "bandwidth (a read stream and a copy) and fp32 atomic-add rate into "
                         "profiles/attainable_peaks.json")
    ap.add_argument("--groups", type=int, default=7,
                    help="groups of 20 back-to-back calls for the pages' statistic (0: none, e.g. "
                         "under a profiler)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/<kernel>_<workload>.md from rocprofv3 kernel traces under "
                         "DIR (trace_<workload>/ with the bench.py line in bench_<workload>.json); "
                         "no GPU needed")
    ap.add_argument("--no-variants", dest="variants", action="store_false",
                    help="default workload only: skip the other configurations under 'variants'")
    ap.add_argument("--replicas", type=int, default=3,
                    help="decode: also time calls that rotate over this many copies of the inputs "
                         "(cold Infinity Cache); 0 disables")
    ap.add_argument("--splits", type=int, default=1,
                    help="decode workloads: time the split-KV path with this many splits as the "
                         "main line (1: the unsplit path)")
    ap.add_argument("--big-pool-gib", type=float, default=0.0,
                    help="decode: also time the same call with its pages scattered over a pool of "
                         "this many GiB (above 4 GiB the kernels rebase a resource per copied row)")
    return ap.parse_args()


def big_pool_case(case, gib, dev, seed=11):
    """The decode case with its pages moved to random pages of a pool of
    `gib` GiB on `dev` (the pool's other pages are zero and never read), the
    block table remapped to match."""
    import dataclasses
    import torch
    n, page, _, d = case.kv_cache.shape
    pages = int(gib * (1 << 30)) // (page * d * 2)
    if pages < n:
        raise ValueError("pool smaller than the case's pages")
    gen = torch.Generator().manual_seed(seed)
    new_page = torch.randperm(pages, generator=gen)[:n].to(torch.int32)
    bt = case.block_table.clone()
    bt[bt >= 0] = new_page[bt[bt >= 0].long()]
    pool = torch.zeros((pages, page, 1, d), dtype=case.kv_cache.dtype, device=dev)
    pool[new_page.long().to(dev)] = case.kv_cache.to(dev)
    return dataclasses.replace(case, name=f"{case.name}_pool{gib:g}gib", kv_cache=pool,
                               block_table=bt)


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------

def make_case(name):
    from sparse_top_mla_amd import workloads as W
    if name == "prefill_h64":
        return W.prefill_h64(with_length=False)
    if name == "prefill_h64_len":
        return W.prefill_h64(with_length=True)
    if name == "prefill_h128":
        return W.prefill_h128()
    if name == "decode_dynamic":
        return W.decode_dynamic(with_length=True)
    if name == "decode_dynamic_nolen":
        return W.decode_dynamic(with_length=False)
    if name == "decode_fixed":
        return W.decode_fixed()
    if name == "decode_fixed_b2":
        # the pages' small-batch run of the fixed top-k shape (B = 2)
        return W.decode_fixed(batch=2)
    if name == "tiny":
        return W.tiny_prefill()
    if name == "bwd_h64":
        # the pages' backward shape: T = 4096, topk = 2048, h_q = 64, d_qk = 576
        return W.bwd_h64()
    if name == "block_sparse_h8":
        # the pages' block-sparse forward benchmark: h = 8, 192/128, sink + 4-block window
        return W.block_sparse_h8()
    raise ValueError(name)


def is_decode(case):
    return hasattr(case, "kv_cache")


def is_block_sparse(case):
    return hasattr(case, "row_ptr")


def bs_counts(case):
    """Block-sparse FLOPs over the selected pairs (2 h_q (192 + 128) per
    (row, key) pair a row attends) and the minimum bytes of one call: q, the
    K and V rows some query block selects (once per KV head), the selection,
    out and lse."""
    s, qbk, kbk = case.s, case.q_block, case.k_block
    ptr, col = case.row_ptr.numpy(), case.col_idx.numpy()
    nk = -(-s // kbk)
    pairs = np.zeros(s, dtype=np.int64)
    named = np.zeros(nk, dtype=bool)
    for qb in range(ptr.size - 1):
        r0, r1 = qb * qbk, min((qb + 1) * qbk, s)
        i = np.arange(r0, r1)
        for b in col[ptr[qb]:ptr[qb + 1]]:
            if not 0 <= b < nk:
                continue
            named[b] = True
            k0, k1 = b * kbk, min((b + 1) * kbk, s)
            pairs[r0:r1] += np.clip(i - k0 + 1, 0, k1 - k0) if case.causal else (k1 - k0)
    h_q, h_kv = case.h_q, case.k.shape[1]
    key_rows = int(sum(min((b + 1) * kbk, s) - b * kbk for b in np.nonzero(named)[0]))
    n_pairs = int(pairs.sum())
    bytes_ = (s * h_q * 192 * 2 + key_rows * h_kv * (192 + 128) * 2 + (ptr.size + col.size) * 4
              + s * h_q * 128 * 2 + s * h_q * 4)
    return dict(flops=2.0 * h_q * (192 + 128) * n_pairs, bytes=float(bytes_), valid_pairs=n_pairs,
                rows=s, valid_per_row=pairs)


def valid_mask(case):
    """[rows, topk] bool: position j of row r is one of the row's keys."""
    idx = case.indices.reshape(-1, case.topk).numpy().astype(np.int64)
    rows = idx.shape[0]
    if is_decode(case):
        mbps = case.block_table.shape[1]
        bound = np.minimum(case.cache_seqlens.numpy().astype(np.int64), mbps * 64)
        bound = np.repeat(bound, case.s_q)
    else:
        bound = np.full(rows, case.s_kv, dtype=np.int64)
    ok = (idx >= 0) & (idx < bound[:, None])
    pos = np.arange(case.topk)[None, :]
    if case.topk_length is not None:
        L = np.clip(case.topk_length.reshape(-1).numpy().astype(np.int64), 0, case.topk)
    else:
        last = np.where(ok, pos, -1).max(axis=1)
        L = last + 1
    ok &= pos < L[:, None]
    if is_decode(case):
        b = np.repeat(np.arange(case.batch), case.s_q)
        bt = case.block_table.numpy().astype(np.int64)
        page = np.where(ok, bt[b[:, None], np.where(ok, idx, 0) // 64], -1)
        ok &= (page >= 0) & (page < case.kv_cache.shape[0])
    return ok, idx


def algorithmic_counts(case):
    """FLOPs over valid keys and the minimum HBM bytes one call must move:
    Q once, every distinct KV row a request names once, the index vectors,
    the optional lengths / block table / cache lengths, and the outputs."""
    ok, idx = valid_mask(case)
    n_valid = int(ok.sum())
    d_qk, d_v, h_q = case.d_qk, case.d_v, case.h_q
    flops = 2.0 * h_q * (d_qk + d_v) * n_valid
    rows = ok.shape[0]
    if is_decode(case):
        b = np.repeat(np.arange(case.batch), case.s_q)
        keys = np.unique(b[:, None].repeat(case.topk, 1)[ok] * (1 << 32) + idx[ok])
        kv_rows = keys.size
        extra = case.block_table.numel() * 4 + case.cache_seqlens.numel() * 4
    else:
        kv_rows = np.unique(idx[ok]).size
        extra = 0
    bytes_ = (rows * h_q * d_qk * 2 + kv_rows * d_qk * 2 + idx.size * 4
              + (rows * 4 if case.topk_length is not None else 0) + extra
              + rows * h_q * d_v * 2 + 2 * rows * h_q * 4)
    return dict(flops=flops, bytes=float(bytes_), valid_pairs=n_valid, kv_rows=int(kv_rows),
                rows=rows, valid_per_row=ok.sum(axis=1))


def bwd_counts(case):
    """Backward FLOPs over valid keys (S = QK^T, dP = dO V^T, dQ = dS K,
    dK = dS^T Q, dV = P^T dO: 2 h_q (3 d_qk + 2 d_v) per valid pair) and the
    minimum HBM bytes of one call: q, out, dout, lse, the index vectors and
    lengths read once, every named KV row read once, dq and the whole dkv
    written once."""
    c = algorithmic_counts(case)
    h_q, d_qk, d_v, rows = case.h_q, case.d_qk, case.d_v, c["rows"]
    c["flops"] = 2.0 * h_q * (3 * d_qk + 2 * d_v) * c["valid_pairs"]
    c["bytes"] = float(rows * h_q * d_qk * 2 + c["kv_rows"] * d_qk * 2 + case.indices.numel() * 4
                       + (rows * 4 if case.topk_length is not None else 0)
                       + 2 * rows * h_q * d_v * 2 + rows * h_q * 4
                       + rows * h_q * d_qk * 2 + case.s_kv * d_qk * 2)
    return c


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
#
# A timed step is one call of the library's C entry point with every argument
# marshalled beforehand (inputs and outputs resident on the device): the
# Python binding's per-call checks cost tens of microseconds, as much as a
# decode kernel, and are not part of the hot path.  The first call of every
# workload goes through the binding, which validates the shapes.

def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _checked(lib, fn, args):
    def call():
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"status {st}: {lib.sparse_mla_last_error().decode()}")
    return call


def gpu_call_bs(case, dev):
    """One block-sparse forward call with every input resident on `dev`."""
    import torch
    import sparse_top_mla_amd as smla
    lib = smla.load_library()
    q, k, v, rp, ci = (x.to(dev) for x in (case.q, case.k, case.v, case.row_ptr, case.col_idx))
    out, lse = smla.block_sparse_fwd(q, k, v, rp, ci, case.q_block, case.k_block, case.sm_scale,
                                     causal=case.causal)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (_vp(q), _vp(k), _vp(v), _vp(rp), _vp(ci) if ci.numel() else None, case.s, case.h_q,
            k.shape[1], 192, 128, case.q_block, case.k_block, int(bool(case.causal)),
            ctypes.c_float(case.sm_scale), _vp(out), _vp(lse), stream)
    keep = (q, k, v, rp, ci, out, lse)
    call = _checked(lib, lib.sparse_mla_block_sparse_fwd, args)
    call.keep = keep
    return call


def gpu_call_bwd(case, dev):
    """One backward call with every input resident on `dev`: out and lse come
    from the library's forward on the same inputs (run once, untimed), dout
    is seeded; workspace and outputs are allocated here, outside the call."""
    import torch
    import sparse_top_mla_amd as smla
    from sparse_top_mla_amd import workloads as W
    lib = smla.load_library()
    t = lambda x: None if x is None else x.to(dev)  # noqa: E731
    q, kv, idx = t(case.q), t(case.kv), t(case.indices)
    sink, tl = t(case.attn_sink), t(case.topk_length)
    out, lse, _ = smla.fwd(q, kv, idx, case.sm_scale, case.d_v, attn_sink=sink, topk_length=tl)
    dout = t(W.bwd_dout(case, seed=8))
    ws = torch.empty(smla.bwd_workspace_bytes(case.s_q, case.s_kv, case.d_qk), dtype=torch.uint8,
                     device=dev)
    dq, dkv, _ = smla.bwd(q, kv, out, dout, idx, lse, case.sm_scale, case.d_v, attn_sink=sink,
                          topk_length=tl, workspace=ws)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (_vp(q), _vp(kv), _vp(out), _vp(dout), _vp(idx), _vp(tl), _vp(lse), _vp(sink),
            case.s_q, case.s_kv, case.h_q, 1, case.d_qk, case.d_v, case.topk,
            ctypes.c_float(case.sm_scale), 0, _vp(ws), ws.numel(), _vp(dq), _vp(dkv), None, stream)
    call = _checked(lib, lib.sparse_mla_bwd, args)
    call.keep = (q, kv, idx, sink, tl, out, lse, dout, ws, dq, dkv)
    return call


def gpu_call(case, dev, num_splits=1):
    """One call of the workload on `dev` with its inputs resident there;
    decode with num_splits > 1 runs the split-KV path (workspace allocated
    here, outside the call)."""
    import torch
    import sparse_top_mla_amd as smla
    lib = smla.load_library()
    t = lambda x: None if x is None else x.to(dev)  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    scale = ctypes.c_float(case.sm_scale)
    if is_decode(case):
        q, kvc, bt, cs, idx = (t(case.q), t(case.kv_cache), t(case.block_table),
                               t(case.cache_seqlens), t(case.indices))
        sink, tl = t(case.attn_sink), t(case.topk_length)
        B, s_q, h_q, d_qk = q.shape
        common = (_vp(q), _vp(kvc), _vp(bt), _vp(cs), _vp(idx), _vp(tl), _vp(sink), B, s_q, h_q, 1,
                  d_qk, case.d_v, case.topk, kvc.shape[0], kvc.shape[1], bt.shape[1], scale)
        if num_splits > 1:
            ws = torch.empty(smla.decode_split_workspace_bytes(B, s_q, h_q, case.d_v, num_splits),
                             dtype=torch.uint8, device=dev)
            out, lse, ml = smla.decode_fwd_split(q, kvc, bt, cs, idx, case.sm_scale, num_splits,
                                                 case.d_v, attn_sink=sink, topk_length=tl,
                                                 workspace=ws)
            args = common + (num_splits, _vp(ws), ws.numel(), _vp(out), _vp(lse), _vp(ml), stream)
            call = _checked(lib, lib.sparse_mla_decode_fwd_split, args)
            call.keep = (q, kvc, bt, cs, idx, sink, tl, ws, out, lse, ml)
            return call
        out, lse, ml = smla.decode_fwd(q, kvc, bt, cs, idx, case.sm_scale, case.d_v,
                                       attn_sink=sink, topk_length=tl)
        args = common + (_vp(out), _vp(lse), _vp(ml), stream)
        call = _checked(lib, lib.sparse_mla_decode_fwd, args)
        call.keep = (q, kvc, bt, cs, idx, sink, tl, out, lse, ml)
        return call
    q, kv, idx = t(case.q), t(case.kv), t(case.indices)
    sink, tl = t(case.attn_sink), t(case.topk_length)
    out, lse, ml = smla.fwd(q, kv, idx, case.sm_scale, case.d_v, attn_sink=sink, topk_length=tl)
    s_q, h_q, d_qk = q.shape
    args = (_vp(q), _vp(kv), _vp(idx), _vp(tl), _vp(sink), s_q, kv.shape[0], h_q, 1, d_qk,
            case.d_v, case.topk, scale, _vp(out), _vp(lse), _vp(ml), stream)
    call = _checked(lib, lib.sparse_mla_fwd, args)
    call.keep = (q, kv, idx, sink, tl, out, lse, ml)
    return call


def time_steps(call, steps, warmup):
    """W untimed calls, then exactly K calls between two synchronisations.
    Returns the wall time per call and the per-call time of the events that
    bracket the K calls on the launch stream (the calls queue back to back,
    so this is the kernels' time)."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return wall_ms / steps, a.elapsed_time(b) / steps


def time_groups(call, groups=7, per_group=20):
    """The pages' statistic (FlashMLA PR #216, "Kernel performance"): groups
    of back-to-back calls, each bracketed by events; returns the group means
    in ms."""
    import torch
    stream = torch.cuda.current_stream()
    means = []
    for _ in range(groups):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(per_group):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        means.append(a.elapsed_time(b) / per_group)
    return means


# ---------------------------------------------------------------------------
# CPU baseline (the oracle as it stands, on a bounded row sample)
# ---------------------------------------------------------------------------

def host_threads():
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(case, counts, target_s):
    import oracle
    rows = counts["rows"]
    per_row = counts["valid_per_row"]
    threads = host_threads()

    def run(sel):
        t0 = time.perf_counter()
        if is_decode(case):
            oracle.sparse_mla_decode_fwd(case.q, case.kv_cache, case.block_table, case.cache_seqlens,
                                         case.indices, case.sm_scale, case.d_v,
                                         attn_sink=case.attn_sink, topk_length=case.topk_length,
                                         rows=sel, threads=threads)
        else:
            oracle.sparse_mla_fwd(case.q, case.kv, case.indices, case.sm_scale, case.d_v,
                                  attn_sink=case.attn_sink, topk_length=case.topk_length,
                                  rows=sel, threads=threads)
        return time.perf_counter() - t0

    def sample(n):
        n = max(1, min(rows, n))
        return np.unique(np.linspace(0, rows - 1, n).round().astype(np.int64))

    probe = sample(2 * threads)
    t = run(probe)
    flops_per_s = 2.0 * case.h_q * (case.d_qk + case.d_v) * per_row[probe].sum() / max(t, 1e-9)
    avg_row_flops = 2.0 * case.h_q * (case.d_qk + case.d_v) * per_row.mean()
    n = int(target_s * flops_per_s / max(avg_row_flops, 1.0))
    sel = sample(n)
    t = run(sel)
    flops = 2.0 * case.h_q * (case.d_qk + case.d_v) * per_row[sel].sum()
    return {"value": float(flops / t / 1e12), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{sel.size} of {rows} rows, evenly spaced ({flops / counts['flops']:.2%} of "
                      f"the valid-key FLOPs), {t:.1f} s, fp64 C oracle",
            "seconds": t, "ms_per_call_extrapolated": float(t * counts["flops"] / flops * 1e3)}


def cpu_baseline_bs(case, counts, target_s):
    """The block-sparse oracle on an evenly spaced row sample."""
    import oracle
    rows = counts["rows"]
    per_row = counts["valid_per_row"]
    threads = host_threads()
    pair_flops = 2.0 * case.h_q * (192 + 128)

    def run(sel):
        t0 = time.perf_counter()
        oracle.block_sparse_fwd(case.q, case.k, case.v, case.row_ptr, case.col_idx, case.q_block,
                                case.k_block, case.sm_scale, causal=case.causal, rows=sel,
                                threads=threads)
        return time.perf_counter() - t0

    def sample(n):
        n = max(1, min(rows, n))
        return np.unique(np.linspace(0, rows - 1, n).round().astype(np.int64))

    probe = sample(8 * threads)
    t = run(probe)
    rate = pair_flops * per_row[probe].sum() / max(t, 1e-9)
    n = int(target_s * rate / max(pair_flops * per_row.mean(), 1.0))
    sel = sample(n)
    t = run(sel)
    flops = pair_flops * per_row[sel].sum()
    return {"value": float(flops / t / 1e12), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{sel.size} of {rows} rows, evenly spaced, {t:.1f} s, fp64 C oracle",
            "seconds": t}


def cpu_baseline_bwd(case, counts, target_s):
    """The backward oracle's dq (S, dP and dQ of each pair: 2 h_q (2 d_qk +
    d_v) FLOPs) on an evenly spaced row sample, with seeded stand-ins for out
    and lse."""
    import oracle
    from sparse_top_mla_amd import workloads as W
    rows = counts["rows"]
    per_row = counts["valid_per_row"]
    threads = host_threads()
    dout = W.bwd_dout(case, seed=8)
    out, lse = W.bwd_synthetic_stats(case, seed=9)
    pair_flops = 2.0 * case.h_q * (2 * case.d_qk + case.d_v)

    def run(sel):
        t0 = time.perf_counter()
        oracle.sparse_mla_bwd(case.q, case.kv, out, dout, case.indices, lse, case.sm_scale,
                              case.d_v, attn_sink=case.attn_sink, topk_length=case.topk_length,
                              rows=sel, want_dkv=False, threads=threads)
        return time.perf_counter() - t0

    def sample(n):
        n = max(1, min(rows, n))
        return np.unique(np.linspace(0, rows - 1, n).round().astype(np.int64))

    probe = sample(2 * threads)
    t = run(probe)
    rate = pair_flops * per_row[probe].sum() / max(t, 1e-9)
    n = int(target_s * rate / max(pair_flops * per_row.mean(), 1.0))
    sel = sample(n)
    t = run(sel)
    flops = pair_flops * per_row[sel].sum()
    return {"value": float(flops / t / 1e12), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"dq of {sel.size} of {rows} rows, evenly spaced (S, dP, dQ FLOPs), "
                      f"{t:.1f} s, fp64 C oracle",
            "seconds": t}


# ---------------------------------------------------------------------------
# roofline
# ---------------------------------------------------------------------------

def kernel_file(workload):
    """Source file of the workload's dominant kernel."""
    return {"bwd_h64": "sparse_mla_bwd.hip",
            "block_sparse_h8": "block_sparse_fwd.hip"}.get(workload, "sparse_mla.hip")


def kernel_name(workload):
    """Name fragment of the workload's dominant kernel in rocprofv3 records."""
    return {"bwd_h64": "sparse_mla_bwd_dkv_kernel",
            "block_sparse_h8": "block_sparse_fwd"}.get(workload, "sparse_mla_fwd")


def call_kernels(workload):
    """Name fragments of the kernels whose counters one call adds up: the
    dominant kernel, and for the backward also its row pass."""
    if workload == "bwd_h64":
        return ["sparse_mla_bwd_dkv_kernel", "sparse_mla_bwd_kernel<"]
    return [kernel_name(workload)]


def kernel_source_digest(workload=None):
    """Digest of the device code (the source above its host-side section)
    without comments and blank lines, so that stored counter figures stay
    attached to the kernels they were taken on; host-side validation and
    dispatch changes do not touch them."""
    import re
    src = (ROOT / "sparse_top_mla_amd" / "csrc" / kernel_file(workload)).read_text()
    cut = src.find("\n// host side\n")
    if cut >= 0:
        src = src[:cut]
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def stored_counters(workload):
    """The committed rocprofv3 counter record of this workload, if it was
    taken on the current kernel source (else None)."""
    f = PROFILES / f"traffic_{workload}.json"
    if not f.exists():
        return None
    rec = json.loads(f.read_text())
    if rec.get("kernel_source_sha256_16") != kernel_source_digest(workload):
        return None
    return rec


def stored_traffic(workload):
    """HBM bytes per launch from the committed counter record, or None."""
    rec = stored_counters(workload)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def roofline(workload, case, counts, kernel_ms):
    if is_decode(case):
        achieved = counts["bytes"] / (kernel_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": stored_traffic(workload)}
    achieved = counts["flops"] / (kernel_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": stored_traffic(workload)}


def _counter_values(csv_path, kernel_substr):
    """Counter values of the dispatches of the first kernel whose name holds
    kernel_substr (the default prefill run also times a second variant)."""
    import csv
    vals, name = [], None
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                name = name or r["Kernel_Name"]
                if r["Kernel_Name"] == name:
                    vals.append(float(r["Counter_Value"]))
    return vals


def ingest_counters(d):
    """HBM bytes per launch of the attention kernel from rocprofv3 counter runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the
    same counter reads for a plain 1 GiB device copy (reads 1 GiB, writes
    1 GiB); the factors are stored with the result."""
    d = Path(d)
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = _counter_values(d / f"pmc_copy_{c}" / "run_counter_collection.csv", "copyBuffer")
        if not v:
            raise SystemExit(f"no copy kernel in pmc_copy_{c}")
        cal[c] = (1 << 30) / (statistics.fmean(v) * 1024.0)
    for sub in sorted(d.glob("pmc_*_FETCH_SIZE")):
        w = sub.name[len("pmc_"):-len("_FETCH_SIZE")]
        if w == "copy":
            continue
        digest = kernel_source_digest(w)
        f = [_counter_values(sub / "run_counter_collection.csv", k) for k in call_kernels(w)]
        wr = [_counter_values(d / f"pmc_{w}_WRITE_SIZE" / "run_counter_collection.csv", k)
              for k in call_kernels(w)]
        if not all(f) or not all(wr):
            continue
        # Per call: the sum over the call's kernels of each one's mean per dispatch.
        fetch = sum(statistics.fmean(v) for v in f) * 1024.0 * cal["FETCH_SIZE"]
        write = sum(statistics.fmean(v) for v in wr) * 1024.0 * cal["WRITE_SIZE"]
        rec = {"workload": w, "hbm_bytes_per_launch": fetch + write,
               "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
               "kernels": call_kernels(w),
               "fetch_kib_raw_mean": [statistics.fmean(v) for v in f],
               "write_kib_raw_mean": [statistics.fmean(v) for v in wr],
               "dispatches": [[len(v) for v in f], [len(v) for v in wr]],
               "copy_calibration_factor": {"FETCH_SIZE": cal["FETCH_SIZE"], "WRITE_SIZE": cal["WRITE_SIZE"]},
               "command": f"rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> -o run --output-format csv -- "
                          f"python3 -u bench.py --workload {w} --no-variants --groups 0 --steps 3 --warmup 1 --cpu-seconds 0 --replicas 0; "
                          f"calibration: ... -- python3 -u bench.py --calibrate-copy",
               "kernel_source_sha256_16": digest}
        busy = _mfma_busy(d / f"pmc_{w}_MFMA", call_kernels(w))
        if busy is not None:
            rec.update(busy)
        PROFILES.mkdir(exist_ok=True)
        (PROFILES / f"traffic_{w}.json").write_text(json.dumps(rec, indent=1) + "\n")
        print(f"{w}: {rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch "
              f"(fetch {fetch / 1e6:.1f}, write {write / 1e6:.1f})")
    write_counter_summary(d, cal)


def write_counter_summary(d, cal):
    """profiles/counters_summary.md: the traffic and MFMA-busy records of
    every workload beside the kernel time of the same workload's trace run
    (bench_<workload>.json under `d`, the pages' group statistic)."""
    rows = []
    for f in sorted(PROFILES.glob("traffic_*.json")):
        rec = json.loads(f.read_text())
        w = rec["workload"]
        if rec.get("kernel_source_sha256_16") != kernel_source_digest(w):
            continue
        bench_f = Path(d) / f"bench_{w}.json"
        ms = alg = None
        if bench_f.exists():
            line = json.loads(bench_f.read_text().strip().splitlines()[-1])
            ms = line["kernel_ms"].get("group_median")
            alg = line["config"]["algorithmic_bytes_per_call"]
        rows.append((w, rec, ms, alg))
    out = ["# HBM traffic and MFMA busy of each workload's dominant kernel", "",
           "Per workload, one rocprofv3 run per counter pass (FETCH_SIZE; WRITE_SIZE; "
           "SQ_VALU_MFMA_BUSY_CYCLES with GRBM_GUI_ACTIVE), from the repository root with "
           "`export TMPDIR=/tmp`:", "", "```",
           "rocprofv3 --pmc <counters> -d <dir>/pmc_<workload>_<FETCH_SIZE|WRITE_SIZE|MFMA> -o run "
           "--output-format csv -- python3 -u bench.py --workload <workload> --no-variants --groups 0 "
           "--steps 3 --warmup 1 --cpu-seconds 0 --replicas 0",
           "rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> -d <dir>/pmc_copy_<counter> -o run --output-format "
           "csv -- python3 -u bench.py --calibrate-copy",
           "python3 bench.py --ingest-counters <dir>", "```", "",
           f"A plain 1 GiB device copy calibrates the counters: FETCH_SIZE x {cal['FETCH_SIZE']:.4f}, "
           f"WRITE_SIZE x {cal['WRITE_SIZE']:.4f}.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
           "((GRBM_GUI_ACTIVE / XCDs) x SIMDs).  The kernel time is the median of 7 group means of 20 "
           "calls from the trace run of the same workload "
           "(`rocprofv3 --kernel-trace --stats ... bench.py --workload <workload> --no-variants`).", "",
           "| workload | HBM bytes per launch | algorithmic bytes | ratio | HBM GB/s at the kernel time | "
           "MFMA busy | kernel time (group median) |", "|---|---|---|---|---|---|---|"]
    for w, rec, ms, alg in rows:
        b = rec["hbm_bytes_per_launch"]
        gbs = f"{b / (ms * 1e-3) / 1e9:.0f}" if ms else "-"
        ratio = f"{b / alg:.2f}" if alg else "-"
        algs = f"{alg / 1e6:.1f} MB" if alg else "-"
        busy = f"{rec['mfma_busy_frac']:.3f}" if "mfma_busy_frac" in rec else "-"
        t = f"{ms * 1e3:.1f} us" if ms else "-"
        out.append(f"| {w} | {b / 1e6:.1f} MB | {algs} | {ratio} | {gbs} | {busy} | {t} |")
    out += ["", "FETCH_SIZE counts L2 -> fabric reads, so KV rows served by the 256 MB Infinity Cache "
            "after an L2 miss count as fetched bytes too: the prefill KV tables (8.4 MB, 4.7 MB) fit "
            "the Infinity Cache but not one XCD's 4 MB L2, which is why prefill fetches 2-3x its "
            "algorithmic bytes.  The decode pools (1.2 GB and more) do not fit it."]
    (PROFILES / "counters_summary.md").write_text("\n".join(out) + "\n")
    print("wrote profiles/counters_summary.md")


def _mfma_busy(sub, kernels=("sparse_mla_fwd",)):
    """MFMA-busy fraction of a call's kernels from one rocprofv3 run with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE.  The SQ counter sums busy
    cycles over every SIMD; GRBM_GUI_ACTIVE sums the active cycles of every
    XCD; the agent record gives the SIMD and XCD counts:
        busy = MFMA_BUSY / ((GUI_ACTIVE / Num_Xcc) * Simd_Count),
    each summed over the call's kernels (means per dispatch)."""
    import csv
    f = sub / "run_counter_collection.csv"
    a = sub / "run_agent_info.csv"
    if not f.exists() or not a.exists():
        return None
    simd = xcc = None
    with open(a) as fh:
        for r in csv.DictReader(fh):
            if r.get("Name", "").startswith("gfx"):
                simd, xcc = int(r["Simd_Count"]), int(r["Num_Xcc"])
    with open(f) as fh:
        all_rows = list(csv.DictReader(fh))
    busy = gui = 0.0
    for kernel in kernels:
        rows = [r for r in all_rows if kernel in r["Kernel_Name"]]
        if not rows or not simd:
            return None
        name = rows[0]["Kernel_Name"]
        vals = {}
        for r in rows:
            if r["Kernel_Name"] == name:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        busy += statistics.fmean(vals["SQ_VALU_MFMA_BUSY_CYCLES"])
        gui += statistics.fmean(vals["GRBM_GUI_ACTIVE"])
    return {"mfma_busy_frac": busy / ((gui / xcc) * simd),
            "mfma_busy_cycles_mean": busy, "grbm_gui_active_mean": gui,
            "mfma_busy_command": f"rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -o run "
                                 f"--output-format csv -- python3 -u bench.py --workload "
                                 f"{sub.name[len('pmc_'):-len('_MFMA')]} --no-variants --groups 0 --steps 3 --warmup 1 --cpu-seconds 0 --replicas 0"}


TRACE_COMMAND = ("rocprofv3 --kernel-trace --stats -d <dir>/trace_{w} -o run --output-format csv -- "
                 "python3 -u bench.py --workload {wl} --no-variants --cpu-seconds 0 --replicas 0{extra}")


def summarize_traces(d):
    """profiles/<kernel>_<workload>.md from the rocprofv3 kernel trace of one
    bench.py run per workload: the per-kernel statistics, the dominant
    kernel's timed region (its last `steps` dispatches before the group
    calls) and the bench.py line of the same run."""
    import csv
    import re
    d = Path(d)
    for sub in sorted(d.glob("trace_*")):
        w = sub.name[len("trace_"):]
        # trace_<workload>_split<N>: the split-KV path (bench.py --splits N)
        m = re.match(r"^(.*)_split(\d+)$", w)
        wl, extra = (m.group(1), f" --splits {m.group(2)}") if m else (w, "")
        stats_f, trace_f = sub / "run_kernel_stats.csv", sub / "run_kernel_trace.csv"
        bench_f = d / f"bench_{w}.json"
        if not stats_f.exists() or not trace_f.exists() or not bench_f.exists():
            continue
        line = json.loads(bench_f.read_text().strip().splitlines()[-1])
        stats = [r for r in csv.DictReader(open(stats_f))
                 if "sparse_mla" in r["Name"] or "block_sparse" in r["Name"] or "combine" in r["Name"]
                 or "row_lengths" in r["Name"] or "dkv" in r["Name"] or "bwd_" in r["Name"]]
        name_frag = kernel_name(wl)
        disp = sorted((r for r in csv.DictReader(open(trace_f)) if name_frag in r["Kernel_Name"]),
                      key=lambda r: int(r["Start_Timestamp"]))
        groups = line.get("kernel_ms", {}).get("group_groups", 0) or 0
        steps = line["steps"]
        timed = disp[len(disp) - groups * 20 - steps:len(disp) - groups * 20] if disp else []
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        kname = disp[0]["Kernel_Name"] if disp else name_frag
        short = kname.replace("(anonymous namespace)::", "").replace("void ", "").split("<")[0]
        out = [f"# {short} — {line['config']['workload']}", "",
               "Command (from the repository root on one MI355X; `export TMPDIR=/tmp` first):", "",
               "```", TRACE_COMMAND.format(w=w, wl=wl, extra=extra), "```", "",
               f"bench.py timed {steps} calls after {line['warmup']} warmups through the C entry point "
               f"(and {groups} groups of 20 calls after them).", "",
               "rocprofv3 kernel statistics (run_kernel_stats.csv):", "",
               "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for r in stats:
            out.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                       f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        if dur:
            out += ["", f"Timed region of `{kname}` (its {len(dur)} dispatches of the timed steps in "
                        f"run_kernel_trace.csv): mean {statistics.fmean(dur):.1f} us, median "
                        f"{statistics.median(dur):.1f} us."]
        rf = line["roofline"]
        out += ["", "bench.py line of the same run (under the profiler):", "",
                f"- kernel time per call over the timed region: {line['kernel_ms']['timed_region_mean'] * 1e3:.1f} us",
                f"- roofline: {rf['achieved']:.1f} {rf['unit']} of {rf['peak']} ({rf['bound']}), "
                f"frac {rf['frac']:.3f}",
                f"- algorithmic bytes per call {line['config']['algorithmic_bytes_per_call'] / 1e6:.1f} MB, "
                f"FLOPs per call {line['config']['flops_per_call']:.4g}"]
        fname = PROFILES / f"{short}_{w}.md"
        PROFILES.mkdir(exist_ok=True)
        fname.write_text("\n".join(out) + "\n")
        print(f"wrote {fname.relative_to(ROOT)}")


def attainable_peaks():
    """This device's attainable dense bf16 MFMA rate (an MFMA loop on every
    SIMD) and HBM bandwidth, both from the benchmark's probe library: a
    read-only stream over 4 GiB (the rate a read-dominated kernel such as the
    decode gather can attain) and a device copy of 4 GiB (reads and writes
    counted)."""
    import torch
    lib = ctypes.CDLL(str(ROOT / "sparse_top_mla_amd" / "libsmla_probe.so"))
    lib.smla_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.smla_probe_mfma_count.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.smla_probe_mfma_count.restype = ctypes.c_longlong
    lib.smla_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(0)
    blocks, iters = props.multi_processor_count * 4, 4096
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    launch = lambda: lib.smla_probe_mfma(out.data_ptr(), blocks, iters, stream)  # noqa: E731
    assert launch() == 0
    mfma_ms = statistics.median(time_groups(launch, groups=7, per_group=3))
    flops = lib.smla_probe_mfma_count(blocks, iters) * 2.0 * 32 * 32 * 16
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_()
    rblocks = props.multi_processor_count * 64
    words = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda:0")
    read = lambda: lib.smla_probe_stream_read(src.data_ptr(), n, words.data_ptr(), rblocks, stream)  # noqa: E731
    assert read() == 0
    read_ms = statistics.median(time_groups(read, groups=7, per_group=3))
    dst = torch.empty_like(src)
    copy_ms = statistics.median(time_groups(lambda: dst.copy_(src), groups=7, per_group=3))
    del src, dst
    lib.smla_probe_atomic_add.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.smla_probe_atomic_count.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.smla_probe_atomic_count.restype = ctypes.c_longlong
    arows, ablocks, aiters = 4096, props.multi_processor_count * 8, 128
    acc = torch.zeros(arows * 576, dtype=torch.float32, device="cuda:0")
    atom = lambda: lib.smla_probe_atomic_add(acc.data_ptr(), arows, ablocks, aiters, stream)  # noqa: E731
    assert atom() == 0
    atom_ms = statistics.median(time_groups(atom, groups=7, per_group=3))
    adds = lib.smla_probe_atomic_count(ablocks, aiters)
    return {"mfma_tflops": flops / (mfma_ms * 1e-3) / 1e12,
            "hbm_read_gbs": n / (read_ms * 1e-3) / 1e9,
            "hbm_gbs": 2.0 * n / (copy_ms * 1e-3) / 1e9,
            "atomic_add_gps": adds / (atom_ms * 1e-3) / 1e9,
            "atomic_probe": f"{ablocks} workgroups of 256 threads x {aiters} x 9 fp32 "
                            f"global_atomic_add_f32 (4 hashed rows x 16 words per instruction) "
                            f"into a [{arows}][576] accumulator, median of 7 group means of 3 "
                            f"launches: {atom_ms:.3f} ms",
            "mfma_probe": f"{blocks} workgroups x 8 waves x {iters} x 4 independent "
                          f"v_mfma_f32_32x32x16_bf16, median of 7 group means of 3 launches: "
                          f"{mfma_ms:.3f} ms",
            "read_probe": f"read-only stream of {n >> 30} GiB, {rblocks} workgroups of 256 "
                          f"threads, median of 7 group means of 3 launches: {read_ms:.3f} ms",
            "copy_probe": f"torch device copy of {n >> 30} GiB (read + write), median of 7 group "
                          f"means of 3: {copy_ms:.3f} ms",
            "device": props.name, "command": "python3 bench.py --attainable"}


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB (reads 1 GiB, writes 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def measure(workload, case, dev, steps, warmup, groups=7, num_splits=1):
    """Times one workload: exactly `steps` calls after `warmup` (wall clock and
    events around the timed region), then the pages' 7 groups of 20 calls.
    num_splits > 1 (decode): the split-KV path.  Returns (record, counts)."""
    import torch
    bwd = workload == "bwd_h64"
    bs = is_block_sparse(case)
    counts = bwd_counts(case) if bwd else bs_counts(case) if bs else algorithmic_counts(case)
    call = (gpu_call_bwd(case, dev) if bwd else gpu_call_bs(case, dev) if bs
            else gpu_call(case, dev, num_splits=num_splits))
    torch.cuda.synchronize()
    ms_per_step, kernel_ms = time_steps(call, steps, warmup)
    gm = time_groups(call, groups=groups) if groups > 0 else [kernel_ms]
    rec = {
        "workload": case.name,
        "ms_per_call": ms_per_step,
        "kernel_ms": kernel_ms,
        "group_means_ms": {"median": statistics.median(gm), "min": min(gm),
                           "max": max(gm), "groups": groups, "calls_per_group": 20},
        "tflops": counts["flops"] / (kernel_ms * 1e-3) / 1e12,
        "roofline": roofline(workload, case, counts, kernel_ms),
        "hbm_gbs_algorithmic": counts["bytes"] / (kernel_ms * 1e-3) / 1e9,
        "valid_pairs": counts["valid_pairs"],
        "flops_per_call": counts["flops"],
        "algorithmic_bytes_per_call": counts["bytes"],
    }
    stored = stored_counters(workload)
    if stored is not None:
        if "mfma_busy_frac" in stored:
            rec["rocprof_mfma_busy_frac"] = stored["mfma_busy_frac"]
        if stored.get("hbm_bytes_per_launch"):
            rec["rocprof_hbm_frac"] = stored["hbm_bytes_per_launch"] / (kernel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    del call
    return rec, counts


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.summarize_trace:
        summarize_traces(args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.attainable:
        rec = attainable_peaks()
        PROFILES.mkdir(exist_ok=True)
        (PROFILES / "attainable_peaks.json").write_text(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    case = make_case(args.workload)
    bwd = args.workload == "bwd_h64"
    bs = is_block_sparse(case)
    if args.splits > 1 and not is_decode(case):
        sys.exit("--splits applies to the decode workloads")
    main_rec, counts = measure(args.workload, case, dev, args.steps, args.warmup, args.groups,
                               num_splits=args.splits)
    if args.splits > 1:
        # The stored counter records are the unsplit path's.
        main_rec["roofline"]["traffic"] = None
    value = counts["flops"] / (main_rec["ms_per_call"] * 1e-3) / 1e12

    variants = {}
    if args.workload == "prefill_h64" and args.variants:
        # Every other configuration of the target statement, each measured the
        # same way (the graded decode row is the one with topk_length).
        for w in ("prefill_h64_len", "tiny", "prefill_h128", "decode_dynamic",
                  "decode_dynamic_nolen", "decode_fixed"):
            c = make_case(w)
            rec, _ = measure(w, c, dev, args.steps, args.warmup, args.groups)
            variants[w] = rec
            del c
            torch.cuda.empty_cache()
    if is_decode(case) and args.replicas > 1:
        # Cold variant: rotate over copies of the inputs, so that a call does
        # not find the previous call's KV rows in the Infinity Cache.
        calls = [gpu_call(case, dev) for _ in range(args.replicas)]
        k = [0]

        def rotating():
            calls[k[0] % len(calls)]()
            k[0] += 1
        ms_cold, kms_cold = time_steps(rotating, args.steps, args.warmup)
        variants[f"cold_{args.replicas}_replicas"] = {
            "ms_per_call": ms_cold, "kernel_ms": kms_cold,
            "hbm_gbs_algorithmic": counts["bytes"] / (kms_cold * 1e-3) / 1e9}
        del calls
    if is_decode(case) and args.big_pool_gib > 0:
        big = big_pool_case(case, args.big_pool_gib, dev)
        call_big = gpu_call(big, dev)
        ms_big, kms_big = time_steps(call_big, args.steps, args.warmup)
        import sparse_top_mla_amd as smla
        variants[f"pool_{args.big_pool_gib:g}gib"] = {
            "kernel": smla.last_kernel(), "pool_bytes": big.kv_cache.numel() * 2,
            "ms_per_call": ms_big, "kernel_ms": kms_big,
            "group_means_ms_median": statistics.median(time_groups(call_big)),
            "hbm_gbs_algorithmic": counts["bytes"] / (kms_big * 1e-3) / 1e9}
        del call_big, big
        torch.cuda.empty_cache()
    rows = case.batch * case.s_q if is_decode(case) else counts["rows"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if is_decode(case) and rows < cus and case.h_q == 128 and args.splits == 1:
        # Fewer rows than CUs: the split-KV path, at the binding's split count.
        import sparse_top_mla_amd as smla
        splits = max(2, smla.decode_num_splits(case.batch, case.s_q, case.topk))
        call_split = gpu_call(case, dev, num_splits=splits)
        ms_split, kms_split = time_steps(call_split, args.steps, args.warmup)
        variants[f"split_{splits}"] = {
            "num_splits": splits, "ms_per_call": ms_split, "kernel_ms": kms_split,
            "group_means_ms_median": statistics.median(time_groups(call_split)),
            "hbm_gbs_algorithmic": counts["bytes"] / (kms_split * 1e-3) / 1e9}
        del call_split

    result = {
        "metric": METRIC_BWD if bwd else METRIC_BS if bs else METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": ({
            "workload": case.name, "s": case.s, "h_q": case.h_q, "h_kv": case.k.shape[1],
            "d_qk": 192, "d_v": 128, "q_block": case.q_block, "k_block": case.k_block,
            "causal": case.causal, "selected_blocks": int(case.col_idx.numel()),
            "valid_pairs": counts["valid_pairs"], "flops_per_call": counts["flops"],
            "algorithmic_bytes_per_call": counts["bytes"],
        } if bs else {
            "workload": case.name,
            "rows": counts["rows"],
            "h_q": case.h_q, "d_qk": case.d_qk, "d_v": case.d_v, "topk": case.topk,
            "valid_pairs": counts["valid_pairs"],
            "flops_per_call": counts["flops"],
            "algorithmic_bytes_per_call": counts["bytes"],
            "topk_length": case.topk_length is not None,
            "attn_sink": case.attn_sink is not None,
            **({"num_splits": args.splits} if args.splits > 1 else {}),
        }),
        "kernel_ms": {"timed_region_mean": main_rec["kernel_ms"],
                      **{f"group_{k}": v for k, v in main_rec["group_means_ms"].items()}},
        "roofline": main_rec["roofline"],
        "hbm_gbs_algorithmic": main_rec["hbm_gbs_algorithmic"],
    }
    for k in ("rocprof_mfma_busy_frac", "rocprof_hbm_frac"):
        if k in main_rec:
            result[k] = main_rec[k]
    if variants:
        result["variants"] = variants
    peaks = PROFILES / "attainable_peaks.json"
    if peaks.exists():
        p = json.loads(peaks.read_text())
        att = p.get("hbm_read_gbs", p["hbm_gbs"]) if is_decode(case) else p["mfma_tflops"]
        result["attainable"] = {"mfma_tflops": p["mfma_tflops"], "hbm_copy_gbs": p["hbm_gbs"],
                                "hbm_read_gbs": p.get("hbm_read_gbs"),
                                "frac_of_attainable": result["roofline"]["achieved"] / att}
        if bwd:
            import sparse_top_mla_amd as smla
            result["dkv_path"] = smla.last_kernel()
        if bwd and p.get("atomic_add_gps") and result.get("dkv_path") == "bwd_scatter":
            # The dkv reduction is one fp32 atomic add per valid (row, key)
            # pair and d_qk column: its time at the probe's rate is a floor.
            adds = float(counts["valid_pairs"]) * case.d_qk
            floor_ms = adds / (p["atomic_add_gps"] * 1e9) * 1e3
            result["atomic_bound"] = {"adds_per_call": adds,
                                      "attainable_adds_per_s": p["atomic_add_gps"] * 1e9,
                                      "floor_ms": floor_ms,
                                      "frac": floor_ms / main_rec["kernel_ms"]}
    if args.cpu_seconds > 0 and bwd:
        result["cpu_baseline"] = cpu_baseline_bwd(case, counts, args.cpu_seconds)
    elif args.cpu_seconds > 0 and bs:
        result["cpu_baseline"] = cpu_baseline_bs(case, counts, args.cpu_seconds)
    elif args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(case, counts, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
