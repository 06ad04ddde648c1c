"""Plant plausible mistakes in copies of the oracle source and check that the
pins catch every one of them (CPU only; the real oracle is never modified)."""
import shutil
import subprocess
from pathlib import Path

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, exact text in the oracle source, replacement)
MUTANTS = [
    ("dropped_scale", "s[j] = sm_scale * acc;", "s[j] = acc;"),
    ("length_off_by_one", "if (is_valid_index(idx_row[j], bound)) L = j + 1;",
     "if (is_valid_index(idx_row[j], bound)) L = j;"),
    ("validity_inclusive_bound", "return idx >= 0 && (int64_t)idx < bound;",
     "return idx >= 0 && (int64_t)idx <= bound;"),
    ("validity_admits_negative", "return idx >= 0 && (int64_t)idx < bound;",
     "return idx >= -1 && (int64_t)idx < bound;"),
    ("lse_drops_max", "lse_row[h] = m + log(Z);", "lse_row[h] = log(Z);"),
    ("lse_includes_sink", "lse_row[h] = m + log(Z);", "lse_row[h] = m + log(denom);"),
    ("sink_unshifted", "denom += exp((double)attn_sink[h] - m);", "denom += exp((double)attn_sink[h]);"),
    ("sink_sign", "denom += exp((double)attn_sink[h] - m);", "denom += exp(-(double)attn_sink[h] - m);"),
    ("value_from_tail_columns", "o[c] += p * bf16_to_double(keys[j][c]);",
     "o[c] += p * bf16_to_double(keys[j][c + (d_qk - d_v)]);"),
    ("no_normalisation", "for (int32_t c = 0; c < d_v; ++c) o[c] /= denom;", ""),
    ("head_ignored", "const uint16_t *qh = q_row + (int64_t)h * d_qk;", "const uint16_t *qh = q_row;"),
    ("explicit_length_ignored", "if (explicit_len != NULL) {", "if (0) {"),
    ("explicit_length_unclamped_low", "if (L < 0) L = 0;", ""),
    ("empty_lse_sign", "lse_row[h] = INFINITY;", "lse_row[h] = -INFINITY;"),
    ("empty_max_sign", "ml_row[h] = -INFINITY;", "ml_row[h] = INFINITY;"),
    ("max_logits_unscaled", "ml_row[h] = m;", "ml_row[h] = m / sm_scale;"),
    ("page_slot_wrong", "keys[nk++] = kv_cache + (page * page_size + idx[j] % page_size) * (int64_t)d_qk;",
     "keys[nk++] = kv_cache + (page * page_size + idx[j] / page_size) * (int64_t)d_qk;"),
    ("page_table_row_wrong", "int64_t page = block_table[b * max_blocks_per_seq + idx[j] / page_size];",
     "int64_t page = block_table[idx[j] / page_size];"),
    ("page_range_drops_page_zero", "if (page < 0 || page >= num_blocks) continue;",
     "if (page <= 0 || page >= num_blocks) continue;"),
    ("page_range_drops_last_page", "if (page < 0 || page >= num_blocks) continue;",
     "if (page < 0 || page >= num_blocks - 1) continue;"),
    ("page_range_clamps_instead_of_masking", "if (page < 0 || page >= num_blocks) continue;",
     "if (page < 0 || page >= num_blocks) page = 0;"),
    ("decode_bound_ignored", "if (!is_valid_index(idx[j], bound)) continue;",
     "if (!is_valid_index(idx[j], 1 << 30)) continue;"),
    ("row_bound_not_clamped",
     "int64_t addressable = (int64_t)max_blocks_per_seq * page_size;\n            if (bound > addressable) bound = addressable;",
     "int64_t addressable = (int64_t)max_blocks_per_seq * page_size;"),
    ("row_length_bound_not_clamped", "bound = cache_seqlens[r / rows_per_seq];\n            if (bound > addressable) bound = addressable;",
     "bound = cache_seqlens[r / rows_per_seq];"),
    ("positions_past_length_used", "for (int32_t j = 0; j < L; ++j)\n                if (is_valid_index(idx[j], s_kv))",
     "for (int32_t j = 0; j < topk; ++j)\n                if (is_valid_index(idx[j], s_kv))"),
    ("softmax_not_shifted", "Z += exp(s[j] - m);", "Z += exp(s[j]);"),
    ("bwd_delta_dropped", "double ds = p * (dp - delta[h]);", "double ds = p * dp;"),
    ("bwd_delta_sign", "double ds = p * (dp - delta[h]);", "double ds = p * (dp + delta[h]);"),
    ("bwd_dq_unscaled", "dqh[d] += sm_scale * ds * bf16_to_double(key[d]);",
     "dqh[d] += ds * bf16_to_double(key[d]);"),
    ("bwd_dv_missing", "for (int32_t c = 0; c < d_v; ++c) dkv_row[c] += p * doh[c];", ""),
    ("bwd_dk_from_key", "dkv_row[d] += sm_scale * ds * bf16_to_double(qhd[d]);",
     "dkv_row[d] += sm_scale * ds * bf16_to_double(key[d]);"),
    ("bwd_dp_over_q", "dp += doh[c] * bf16_to_double(key[c]);", "dp += doh[c] * bf16_to_double(qhd[c]);"),
    ("bwd_delta_without_out", "dl += dout[rh * d_v + c] * out[rh * d_v + c];",
     "dl += dout[rh * d_v + c];"),
    ("bwd_sink_ignored", "if (attn_sink != NULL && !isinf(l)) {", "if (0) {"),
    ("bwd_base2_inverted", "double l = lse_base2 ? lse * log(2.0) : lse;",
     "double l = lse_base2 ? lse / log(2.0) : lse;"),
    ("bs_causal_excludes_diagonal", "if (causal && j > i) continue;", "if (causal && j >= i) continue;"),
    ("bs_query_block_halved", "int64_t qb = i / q_block;", "int64_t qb = i / (2 * q_block);"),
    ("bs_kv_head_interleaved", "const int32_t kvh = h / group;", "const int32_t kvh = h % h_kv;"),
    ("bs_lse_drops_max", "lse[n * h_q + h] = m + log(Z);", "lse[n * h_q + h] = log(Z);"),
    ("bs_value_not_weighted", "for (int32_t c = 0; c < d_v; ++c) o[c] += p * bf16_to_double(vr[c]);",
     "for (int32_t c = 0; c < d_v; ++c) o[c] += bf16_to_double(vr[c]);"),
    ("bwd_d_sink_sign", "d_sink[h] -= exp(", "d_sink[h] += exp("),
    ("bwd_length_ignored", "for (int32_t j = 0; j < len[i]; ++j)\n                if (is_valid_index(idx[j], s_kv))",
     "for (int32_t j = 0; j < topk; ++j)\n                if (is_valid_index(idx[j], s_kv))"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique/absent"
    mutated = workdir / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib_path = workdir / f"lib_{name}.so"
    oracle.build(mutated, lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"
