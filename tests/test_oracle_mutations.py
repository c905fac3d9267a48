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
    "sub_becomes_add": ("double_to_half(pu_c - pv_s)", "double_to_half(pu_c + pv_s)"),
    "add_becomes_sub": ("double_to_half(pv_c + pu_s)", "double_to_half(pv_c - pu_s)"),
    "dropped_sin_term": ("double_to_half(pv_c + pu_s)", "double_to_half(pv_c)"),
    "sin_reads_cos_half": ("double s = (double)row[half + i];", "double s = (double)row[i];"),
    "neox_partner_off_by_one": ("v = i + half;", "v = i + half - (i > 0);"),
    "gptj_pair_swapped": ("u = 2 * i;\n      v = 2 * i + 1;", "u = 2 * i + 1;\n      v = 2 * i;"),
    "ties_away_from_zero": ("(rem == 0.5 && (k & 1))", "(rem == 0.5)"),
    "no_subnormal_clamp": ("if (ue < -14) ue = -14;", "if (ue < -15) ue = -15;"),
    "subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "passthrough_zeroed": ("for (int d = 0; d < head_dim; ++d) tmp[d] = x[d];",
                           "for (int d = 0; d < head_dim; ++d) tmp[d] = 0;"),
    "table_batch_ignored": ("int32_t tb = (table_batch == 1) ? 0 : b;", "int32_t tb = 0;"),
    "k_into_v_plane": ("memcpy(cache + cache_row(b, 0, h, pos, hkv, capacity, D), x,",
                       "memcpy(cache + cache_row(b, 1, h, pos, hkv, capacity, D), x,"),
    "k_not_rotated_in_place": ("        rkv_ref_rotate_row(x, x, row, D, R, style);\n        memcpy",
                               "        memcpy"),
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
    "paged_offset_transposed": ("pool + (((size_t)kid * TPP + off) * hkv + h) * D",
                                "pool + (((size_t)kid * TPP + h) * hkv + off % hkv) * D"),
    "capacity_check_inclusive": ("return cos_sin_len > kv_capacity ?", "return cos_sin_len >= kv_capacity ?"),
    "gather_position_past_table": ("st >= rope_states || p >= rope_rows", "st >= rope_states || p > rope_rows"),
    "gather_ignores_state_indices": ("int64_t st = state_indices ? state_indices[q]", "int64_t st = state_indices ? q"),
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
