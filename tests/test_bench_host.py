"""Host-side checks of the benchmark's counter arithmetic (no GPU).

The MFMA-busy fraction and the HBM bytes per launch are derived from
rocprofv3 CSV files; these tests feed synthetic CSVs with known values and
check the formulas, so a mistake in the normalisation cannot hide behind a
plausible-looking number.
"""
import csv
import json

import numpy as np
import pytest

import bench


def _write_csv(path, header, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _agent(path, simd=1024, xcc=8):
    _write_csv(path, ["Name", "Simd_Count", "Num_Xcc", "Cu_Count"],
               [["AMD EPYC", "0", "0", "0"], ["gfx950", str(simd), str(xcc), "256"]])


def test_mfma_busy_fraction(tmp_path):
    sub = tmp_path / "pmc_prefill_h64_MFMA"
    _agent(sub / "run_agent_info.csv")
    k = "void (anonymous namespace)::sparse_mla_fwd_wide_kernel<512, 2, false, false, false>(x)"
    other = "void (anonymous namespace)::sparse_mla_fwd_wide_kernel<512, 2, false, true, false>(x)"
    # 8 XCDs x 1000 active cycles each; 1024 SIMDs busy for 250 cycles each -> 0.25
    rows = []
    for _ in range(3):
        rows.append([k, "SQ_VALU_MFMA_BUSY_CYCLES", str(1024 * 250)])
        rows.append([k, "GRBM_GUI_ACTIVE", str(8 * 1000)])
        rows.append([other, "SQ_VALU_MFMA_BUSY_CYCLES", str(1024 * 999)])  # a second instance: ignored
        rows.append([other, "GRBM_GUI_ACTIVE", str(8 * 1000)])
    _write_csv(sub / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    rec = bench._mfma_busy(sub)
    assert abs(rec["mfma_busy_frac"] - 0.25) < 1e-12


def test_ingest_counters_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", tmp_path / "profiles")
    d = tmp_path / "meas"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "__amd_rocclr_copyBuffer"
    # the copy reads 1 GiB but FETCH_SIZE reports half of it; WRITE_SIZE is exact
    _write_csv(d / "pmc_copy_FETCH_SIZE" / "run_counter_collection.csv", hdr,
               [[copy, "FETCH_SIZE", str(512 * 1024)]])
    _write_csv(d / "pmc_copy_WRITE_SIZE" / "run_counter_collection.csv", hdr,
               [[copy, "WRITE_SIZE", str(1024 * 1024)]])
    k = "void (anonymous namespace)::sparse_mla_fwd_wide_kernel<576, 1, true, true, false>(x)"
    _write_csv(d / "pmc_decode_dynamic_FETCH_SIZE" / "run_counter_collection.csv", hdr,
               [[k, "FETCH_SIZE", "1000"], [k, "FETCH_SIZE", "3000"]])
    _write_csv(d / "pmc_decode_dynamic_WRITE_SIZE" / "run_counter_collection.csv", hdr,
               [[k, "WRITE_SIZE", "500"], [k, "WRITE_SIZE", "500"]])
    bench.ingest_counters(d)
    rec = json.loads((tmp_path / "profiles" / "traffic_decode_dynamic.json").read_text())
    assert abs(rec["fetch_bytes_per_launch"] - 2000 * 1024 * 2.0) < 1e-6
    assert abs(rec["write_bytes_per_launch"] - 500 * 1024 * 1.0) < 1e-6
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_digest()
    assert "mfma_busy_frac" not in rec  # no MFMA run given


@pytest.mark.parametrize("causal", [True, False])
def test_block_sparse_pair_count_is_brute_force(causal):
    """bench.bs_counts counts the (row, key) pairs the block-sparse forward
    attends: brute force over rows, listed blocks and keys."""
    from sparse_top_mla_amd import workloads as W
    case = W.make_block_sparse("count", s=300, h_q=2, h_kv=1, q_block=64, k_block=64,
                               selection="random", seed=3, causal=causal)
    got = bench.bs_counts(case)
    ptr, col = case.row_ptr.numpy(), case.col_idx.numpy()
    per_row = np.zeros(300, dtype=np.int64)
    for i in range(300):
        qb = i // 64
        for b in col[ptr[qb]:ptr[qb + 1]]:
            if 0 <= b < 5:
                per_row[i] += sum(1 for j in range(b * 64, min(b * 64 + 64, 300))
                                  if not causal or j <= i)
    assert np.array_equal(got["valid_per_row"], per_row)
    assert got["flops"] == 2.0 * 2 * (192 + 128) * per_row.sum()


def test_bwd_flops_count_five_products():
    """The backward's FLOPs are 2 h_q (3 d_qk + 2 d_v) per valid pair."""
    from sparse_top_mla_amd import workloads as W
    case = W.bwd_h64(s_q=64, s_kv=64, topk=32)
    c = bench.bwd_counts(case)
    assert c["flops"] == 2.0 * 64 * (3 * 576 + 2 * 512) * c["valid_pairs"]
    assert c["valid_pairs"] == sum(min(i + 1, 32) for i in range(64))
