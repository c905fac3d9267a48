"""Planted mistakes in the oracle must each fail some pin.

Each case copies ``oracle/rkv_oracle.c``, replaces one exact snippet (which
must occur exactly once) with a plausible mistake -- a dropped term, a wrong
sign or index, swapped operands, an off-by-one bound -- builds the copy and
runs every pin against it in a child process.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rkv_oracle.c")

MUTATIONS = {
    "sub_becomes_add": ("w[u] = pu_c - pv_s;", "w[u] = pu_c + pv_s;"),
    "add_becomes_sub": ("w[v] = pv_c + pu_s;", "w[v] = pv_c - pu_s;"),
    "dropped_sin_term": ("w[v] = pv_c + pu_s;", "w[v] = pv_c;"),
    "sin_reads_cos_half": ("double s = (double)row[half + i];", "double s = (double)row[i];"),
    "neox_partner_off_by_one": ("v = i + half;", "v = i + half - (i > 0);"),
    "gptj_pair_swapped": ("u = 2 * i;\n      v = 2 * i + 1;", "u = 2 * i + 1;\n      v = 2 * i;"),
    "ties_away_from_zero": ("(rem == 0.5 && (k & 1))) k += 1;\n  if (k >= 2048)",
                            "(rem == 0.5)) k += 1;\n  if (k >= 2048)"),
    "no_subnormal_clamp": ("if (ue < -14) ue = -14;", "if (ue < -15) ue = -15;"),
    "subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "passthrough_zeroed": ("? rkv_ref_double_to_half(w[d]) : x[d];",
                           "? rkv_ref_double_to_half(w[d]) : 0;"),
    "passthrough_rounded_from_unnormalised": ("(d < R || norm_w) ?", "(d < R) ?"),
    "table_batch_ignored": ("int32_t tb = (table_batch == 1) ? 0 : b;", "int32_t tb = 0;"),
    "k_into_v_plane": ("memcpy(cache + cache_row(b, 0, h, pos, hkv, capacity, D), x,",
                       "memcpy(cache + cache_row(b, 1, h, pos, hkv, capacity, D), x,"),
    "k_not_rotated_in_place": ("        head_row16(x, x, row, D, R, style, k_w, eps);\n        if (!cache8)",
                               "        if (!cache8)"),
    "end_len_off_by_one": ("int64_t slot = (int64_t)end_lens[b] - seq_len + s;\n      int64_t pos = slot;",
                           "int64_t slot = (int64_t)end_lens[b] - seq_len + s + 1;\n      int64_t pos = slot;"),
    "tree_uses_slot_as_position": ("int64_t pos = pos_ids[(size_t)b * seq_len + s];",
                                   "int64_t pos = slot;"),
    "continuous_ignores_table_length": ("if (slot < 0 || slot >= capacity || pos >= table_len) continue;",
                                        "if (slot < 0 || slot >= capacity) continue;"),
    "paged_k_upper_bound": ("kid >= 0 && kid < num_pages", "kid >= 0 && kid <= num_pages"),
    "paged_capacity_bound": ("if (p >= (int64_t)max_pages_per_seq * TPP) continue;",
                             "if (p > (int64_t)max_pages_per_seq * TPP) continue;"),
    "paged_v_plane_lower_bound": ("vid >= num_pages && vid < 2", "vid >= 0 && vid < 2"),
    "paged_inactive_sequence_kept": ("if (q >= batch) continue;", ""),
    "paged_offset_transposed": ("size_t dst = (((size_t)kid * TPP + off) * hkv + h) * D;",
                                "size_t dst = (((size_t)kid * TPP + h) * hkv + off % hkv) * D;"),
    "capacity_check_inclusive": ("return cos_sin_len > kv_capacity ?", "return cos_sin_len >= kv_capacity ?"),
    "gather_position_past_table": ("st >= rope_states || p >= rope_rows", "st >= rope_states || p > rope_rows"),
    "gather_ignores_state_indices": ("int64_t st = state_indices ? state_indices[q]", "int64_t st = state_indices ? q"),
    # fp8 (E4M3) cache variants
    "e4m3_overflow_to_nan": ("if (a >= 448.0) return (uint8_t)(sign | 0x7e);",
                             "if (a >= 464.0) return (uint8_t)(sign | 0x7f);"),
    "e4m3_ties_away_from_zero": ("(rem == 0.5 && (k & 1))) k += 1;\n  if (k >= 16)",
                                 "(rem == 0.5)) k += 1;\n  if (k >= 16)"),
    "e4m3_subnormal_clamp": ("if (ue < -6) ue = -6;", "if (ue < -7) ue = -7;"),
    "e4m3_decode_subnormal": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "e4m3_decode_bias": ("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 9);"),
    "fp8_multiplies_by_scale": ("rkv_ref_double_to_e4m3(w[d] * (double)rcp)",
                                "rkv_ref_double_to_e4m3(w[d] / (double)rcp)"),
    "fp8_k_from_fp16_rounded": ("rkv_ref_double_to_e4m3(w[d] * (double)rcp)",
                                "rkv_ref_double_to_e4m3(rkv_ref_half_to_double(rkv_ref_double_to_half(w[d])) * (double)rcp)"),
    "fp8_k_uses_v_scale": ("store_row8(cache8 + cache_row(b, 0, h, slot, hkv, cap, D), w, D, k_rcp);",
                           "store_row8(cache8 + cache_row(b, 0, h, slot, hkv, cap, D), w, D, v_rcp);"),
    "fp8_k_unrotated": ("      rkv_ref_rotate_row_wide(k, w, row, D, rotary_dim, style);\n",
                        "      widen_row(k, w, D);\n"),
    "fp8_packed_v_into_k_plane": ("store_row8(cache8 + cache_row(b, 1, h, pos, hkv, capacity, D), w, D, v_rcp);",
                                  "store_row8(cache8 + cache_row(b, 0, h, pos, hkv, capacity, D), w, D, v_rcp);"),
    "fp8_paged_v_unscaled": ("          store_row8(pool8 + dst, w, D, v_rcp);",
                             "          store_row8(pool8 + dst, w, D, 1.0f);"),
    # Q/K RMS norm
    "norm_mean_over_d_minus_1": ("ldexp((double)acc, -48) / (double)head_dim;",
                                 "ldexp((double)acc, -48) / (double)(head_dim - 1);"),
    "norm_sum_drops_last_bit": ("ldexp((double)acc, -48) / (double)head_dim;",
                                "ldexp((double)(acc >> 1 << 1), -48) / (double)head_dim;"),
    "norm_eps_dropped": ("1.0 / sqrt(rkv_ref_mean_square(x, head_dim) + eps);",
                         "1.0 / sqrt(rkv_ref_mean_square(x, head_dim));"),
    "norm_eps_outside_sqrt": ("1.0 / sqrt(rkv_ref_mean_square(x, head_dim) + eps);",
                              "1.0 / (sqrt(rkv_ref_mean_square(x, head_dim)) + eps);"),
    "norm_weight_dropped": ("(rkv_ref_half_to_double(x[d]) * r) * (double)weight[d];",
                            "(rkv_ref_half_to_double(x[d]) * r);"),
    "norm_k_uses_q_weight": ("head_row16(x, x, row, D, R, style, k_w, eps);",
                             "head_row16(x, x, row, D, R, style, q_w, eps);"),
    "norm_q_uses_k_weight_calls_2_3": ("               row, D, R, style, q_w, eps);",
                                       "               row, D, R, style, k_w, eps);"),
    "norm_nan_row_ignored": ("if (has_nan) return NAN;", ""),
    # metadata builders
    "delta_len_inclusive": ("if (j < len && pos <= INT32_MAX)", "if (j <= len && pos <= INT32_MAX)"),
    "delta_overflow_unchecked": ("if (j < len && pos <= INT32_MAX)", "if (j < len)"),
    "delta_position_off_by_one": ("int64_t pos = (int64_t)old_lengths[b] + j;",
                                  "int64_t pos = (int64_t)old_lengths[b] + j + 1;"),
    "delta_padding_owner_kept": ("        delta_to_seq[i] = -1;", "        delta_to_seq[i] = b;"),
    "tree_root_parent_zero": ("parent_ids[(size_t)b * verify_size + i] = i - 1;",
                              "parent_ids[(size_t)b * verify_size + i] = i > 0 ? i - 1 : 0;"),
    "tree_depth_off_by_one": ("depths[(size_t)b * verify_size + i] = i;",
                              "depths[(size_t)b * verify_size + i] = i + 1;"),
    "fp8_reciprocal_truncated": ("return (float)(1.0 / (double)scale);",
                                 "return (float)(1.0 / (double)scale) * (1.0f - 0x1p-23f);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"snippet for {name} must occur once"
    src = tmp_path / "rkv_oracle.c"
    src.write_text(text.replace(old, new))
    hdr = os.path.join(ROOT, "oracle", "rkv_oracle.h")
    (tmp_path / "rkv_oracle.h").write_text(open(hdr).read())
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", str(lib), str(src), "-lm"], check=True)
    runner = os.path.join(ROOT, "tests", "pin_runner.py")
    res = subprocess.run([sys.executable, runner, str(lib)], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, f"{name} not caught: {res.stdout}{res.stderr}"
