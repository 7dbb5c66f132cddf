"""The oracle's pins catch plausible mistakes: each case plants one mistake in
a copy of the oracle's C source (on the CPU, in a temporary directory),
builds it, and runs the whole pin suite against it in a child process; some
pin must fail.  The checked-in oracle is never touched.

The mistakes are the ones an implementation of the pages' steps could
plausibly make, in every oracle function: the combine's arithmetic (a fused
multiply-add split, slot order reversed, a -0 start, ties away from even, a
wrong prob index), the counting sort walked backwards, the chunk map's
padding and indexing, the backward scatters and sums, the EP rank order,
partial rounding and fp64 sum, the router's tie-break, normalisation and
gradient, the mask map's row order and dropping, the zero-prob rule, the
mask combine's unfused arithmetic and gradient dot, the scale rows, the
restore's zero tail, and the fp64 -> bf16 rounding.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

_UNPERMUTE_SLOT = (
    "for (int j = 0; j < k; j++) {\n"
    "                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);\n"
    "                float p = probs ? probs[(int64_t)t * k + j] : 1.0f;\n"
    "                acc = fmaf(")

MUTATIONS = [
    ("fma_split",
     "acc = fmaf(p, bf16_to_f32(in[r * H + h]), acc);",
     "acc = p * bf16_to_f32(in[r * H + h]) + acc;"),
    ("slot_order_reversed",
     _UNPERMUTE_SLOT,
     _UNPERMUTE_SLOT.replace("for (int j = 0; j < k; j++) {\n",
                             "for (int jj = 0; jj < k; jj++) {\n"
                             "                int j = k - 1 - jj;\n")),
    ("negative_zero_start",
     "float acc = +0.0f;\n            " + _UNPERMUTE_SLOT,
     "float acc = -0.0f;\n            " + _UNPERMUTE_SLOT),
    ("ties_away_from_even",
     "if (kept & 1u) kept += 1u;    /* exactly halfway: to even        */",
     "kept += 1u;"),
    ("prob_index",
     "float p = probs ? probs[(int64_t)t * k + j] : 1.0f;\n                acc = fmaf(",
     "float p = probs ? probs[(int64_t)t * k] : 1.0f;\n                acc = fmaf("),
    ("row_map_walked_backwards",
     "    for (int64_t i = 0; i < npairs; i++) {\n        int t = pair_token[i];",
     "    for (int64_t ii = 0; ii < npairs; ii++) {\n"
     "        int64_t i = npairs - 1 - ii;\n        int t = pair_token[i];"),
    ("padding_one_group_too_many",
     "int64_t padded = ((n_g + A - 1) / A) * A;",
     "int64_t padded = (n_g / A + 1) * A;"),
    ("chunk_index_transposed",
     "row_map[d] = (int32_t)(src_off[c] + i);",
     "row_map[d] = (int32_t)(src_off[q] + i);"),
    ("act_grad_drops_prob",
     "float prod = g * p;          /* one fp32 rounding */",
     "float prod = g;"),
    ("ep_ranks_reversed",
     "for (int rank = 0; rank < ep_size; rank++) {",
     "for (int rank = ep_size - 1; rank >= 0; rank--) {"),
    ("ep_partials_unrounded",
     "if (bf16_partials) partial = bf16_to_f32(f32_to_bf16_rne(partial));",
     "(void)bf16_partials;"),
    ("grad_sum_overwrites",
     "acc = acc + bf16_to_f32(d_out[r * H + h]);",
     "acc = bf16_to_f32(d_out[r * H + h]);"),
    ("router_ties_to_higher_expert",
     "if (best < 0 || v > bv) { best = e; bv = v; }",
     "if (best < 0 || v >= bv) { best = e; bv = v; }"),
    ("router_weights_unnormalised",
     "double w = exp(lv[j] - lv[0]) / sum;",
     "double w = exp(lv[j] - lv[0]);"),
    ("router_grad_without_dot",
     "w * (dp - dot));",
     "w * dp);"),
    ("mask_map_rows_ascending",
     "return (x->row < y->row) - (x->row > y->row);",
     "return (x->row > y->row) - (x->row < y->row);"),
    ("mask_drop_off_by_one",
     "if (dense[i] >= num_out) dense[i] = -1;",
     "if (dense[i] > num_out) dense[i] = -1;"),
    ("mask_zero_prob_rule_lost",
     "zero_row = p == 0.0f;\n            }\n            for (int h = 0; h < H; h++)",
     "zero_row = 0;\n            }\n            for (int h = 0; h < H; h++)"),
    ("scaled_mask_zero_prob_rule_lost",
     "zero_row = p == 0.0f;\n            }\n            if (zero_row)",
     "zero_row = 0;\n            }\n            if (zero_row)"),
    ("mask_combine_fused",
     "if (merging_probs) v = v * merging_probs[(int64_t)t * E + e];\n                acc = acc + v;",
     "acc = merging_probs ? fmaf(v, merging_probs[(int64_t)t * E + e], acc) : acc + v;"),
    ("mask_grad_dot_uses_product",
     "dot += (double)bf16_to_f32(fwd_in[(int64_t)row * H + h]) * (double)g;",
     "dot += (double)bf16_to_f32(fwd_in[(int64_t)row * H + h]) * (double)prod;"),
    ("scale_row_of_token_zero",
     "copy_bytes(out_scale + r * scale_row_bytes, scale + (int64_t)t * scale_row_bytes,",
     "copy_bytes(out_scale + r * scale_row_bytes, scale,"),
    ("restore_tail_not_zeroed",
     "for (int64_t s = n_act; s < N_cap; s++) {",
     "for (int64_t s = N_cap; s < N_cap; s++) {"),
    ("f64_to_bf16_one_bit_too_many",
     "int qexp = e - 8;",
     "int qexp = e - 9;"),
    ("unpermute_ep_fp64_sum_in_fp32",
     "total64 = total64 + (double)partial;",
     "total64 = (float)(total64 + (double)partial);"),
    ("permute_bwd_prob_gather_index",
     "d_probs[(int64_t)t * k + j] = d_out_probs[r];",
     "d_probs[(int64_t)t * k + j] = d_out_probs[(int64_t)t * k + j];"),
    ("chunk_order_repeat_accepted",
     "if (c < 0 || c >= C || seen[c]) { status = ORC_BAD_CHUNKS; goto done; }",
     "if (c < 0 || c >= C) { status = ORC_BAD_CHUNKS; goto done; }"),
    ("row_map_repeat_accepted",
     "if (row_id_map[slot] != -1) { status = ORC_DUP_EXPERT; break; }",
     ""),
    ("mask_offsets_ignore_dropping",
     "if (expert_offsets) expert_offsets[e] = (int32_t)(num_out >= 0 && row > num_out ? num_out : row);",
     "if (expert_offsets) expert_offsets[e] = (int32_t)row;"),
    ("chunk_map_overflow_accepted",
     "    if (total > N_cap) { status = ORC_OVERFLOW; goto done; }",
     ""),
    ("row_map_bad_expert_accepted",
     "        if (pair_expert[i] < 0 || pair_expert[i] >= E) return ORC_BAD_EXPERT;",
     ""),
    ("mask_unpermuted_probs_zero",
     "unpermuted_probs[(int64_t)t * E + e] = permuted_probs[row];",
     "unpermuted_probs[(int64_t)t * E + e] = 0.0f;"),
    ("pad_probs_from_destination_index",
     "memcpy(out_probs + (int64_t)d * prob_bytes, probs + (int64_t)s * prob_bytes,",
     "memcpy(out_probs + (int64_t)d * prob_bytes, probs + (int64_t)d * prob_bytes,"),
    ("scaled_mask_scale_skipped_on_zero_prob",
     "            if (scale && out_scale && scale_row_bytes > 0)\n"
     "                copy_bytes(out_scale + (int64_t)row * scale_row_bytes,",
     "            if (scale && out_scale && scale_row_bytes > 0 && !zero_row)\n"
     "                copy_bytes(out_scale + (int64_t)row * scale_row_bytes,"),
    ("restore_overflow_accepted",
     "    if (n_act > N_cap) return ORC_OVERFLOW;\n    return restore_copy(",
     "    return restore_copy("),
    ("restore_stale_entry_copied",
     "if (s >= n_act) { status = ORC_BAD_ROW; continue; }",
     "if (s >= N_cap) { status = ORC_BAD_ROW; continue; }"),
    ("restore_stale_entry_unreported",
     "if (s >= n_act) { status = ORC_BAD_ROW; continue; }",
     "if (s >= n_act) continue;"),
    ("permute_rows_of_reversed_tokens",
     "for (int h = 0; h < H; h++) out[r * H + h] = x[(int64_t)t * H + h];",
     "for (int h = 0; h < H; h++) out[r * H + h] = x[(int64_t)(T - 1 - t) * H + h];"),
    ("permute_probs_of_first_slot",
     "            for (int h = 0; h < H; h++) out[r * H + h] = x[(int64_t)t * H + h];\n"
     "            if (probs && out_probs) out_probs[r] = probs[(int64_t)t * k + j];",
     "            for (int h = 0; h < H; h++) out[r * H + h] = x[(int64_t)t * H + h];\n"
     "            if (probs && out_probs) out_probs[r] = probs[(int64_t)t * k];"),
    ("permute_bwd_slots_reversed",
     "                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);\n"
     "                acc = acc + bf16_to_f32(d_out[r * H + h]);",
     "                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, k - 1 - j);\n"
     "                acc = acc + bf16_to_f32(d_out[r * H + h]);"),
    ("router_softmax_without_max",
     "        for (int j = 0; j < k; j++) sum += exp(lv[j] - lv[0]);\n"
     "        for (int j = 0; j < k; j++) {\n"
     "            double w = exp(lv[j] - lv[0]) / sum;",
     "        for (int j = 0; j < k; j++) sum += exp(lv[j]);\n"
     "        for (int j = 0; j < k; j++) {\n"
     "            double w = exp(lv[j]) / sum;"),
    ("ep_ranks_interleaved",
     "if (topk_idx[(int64_t)t * k + j] / per_rank != rank) continue;",
     "if (topk_idx[(int64_t)t * k + j] % ep_size != rank) continue;"),
    ("prob_grad_dot_on_slot_index_row",
     "double a = (double)bf16_to_f32(fwd_in[r * H + h]);",
     "double a = (double)bf16_to_f32(fwd_in[((int64_t)t * k + j) * H + h]);"),
    ("prob_grad_dot_in_fp32",
     "                        dot += a * b;\n"
     "                    }\n"
     "                    d_probs[(int64_t)t * k + j] = (float)dot;",
     "                        dot = (float)(dot + (float)(a * b));\n"
     "                    }\n"
     "                    d_probs[(int64_t)t * k + j] = (float)dot;"),
    ("mask_prob_grad_dot_in_fp32",
     "dot += (double)bf16_to_f32(fwd_in[(int64_t)row * H + h]) * (double)g;",
     "dot = (float)(dot + (float)((double)bf16_to_f32(fwd_in[(int64_t)row * H + h]) * (double)g));"),
    ("bf16_widening_drops_sign",
     "uint32_t u = ((uint32_t)b) << 16;",
     "uint32_t u = ((uint32_t)(b & 0x7FFFu)) << 16;"),
]

_RUNNER = (
    "import sys; sys.path.insert(0, sys.argv[1]); import oracle; oracle._LIB = sys.argv[2]; "
    "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', sys.argv[3]]))")


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(ORACLE_C).read()
    assert src.count(old) == 1, f"{name}: the line to change is not unique in the oracle"
    mutant_c = tmp_path / "moe_oracle.c"
    mutant_c.write_text(src.replace(old, new, 1))
    mutant_so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                           "-fopenmp", "-shared", "-fPIC", str(mutant_c), "-o", str(mutant_so),
                           "-lm"])
    r = subprocess.run([sys.executable, "-c", _RUNNER, ROOT, str(mutant_so), PINS],
                       capture_output=True, text=True, timeout=600, cwd=str(tmp_path))
    assert r.returncode == 1, (
        f"{name}: no pin failed (exit {r.returncode})\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")
