"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (a dropped term, a wrong sign, index or
operand), builds the copy with gcc on the CPU and runs the pin tests against it in a
subprocess; the pins must fail. The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, mistaken text, replace every occurrence?)
MUTANTS = [
    ("partial_block_mean_over_P", "for (int d = 0; d < a->D; ++d) S[d] /= (double)n;",
     "for (int d = 0; d < a->D; ++d) S[d] /= (double)a->P;", False),
    ("index_query_sum_not_mean", "qidx[d] = acc / (double)G;", "qidx[d] = acc;", False),
    ("score_wrong_operand_index", "acc += qidx[d] * Sj[d];", "acc += qidx[d] * Sj[0];", False),
    ("order_sign_flipped", "if (x->s > y->s) return -1;", "if (x->s > y->s) return 1;", False),
    ("tie_break_reversed", "return (x->j > y->j) - (x->j < y->j);",
     "return (x->j < y->j) - (x->j > y->j);", False),
    ("no_ascending_output", "qsort(out, (size_t)keff, sizeof(int32_t), ascending_i32);", "", False),
    ("logit_scale_dropped", "z[ntok] = a->scale * acc;", "z[ntok] = acc;", False),
    ("index_query_wrong_heads", "for (int h = g * G; h < (g + 1) * G; ++h)\n            acc +=",
     "for (int h = g; h < g + G; ++h)\n            acc +=", False),
    ("length_ignored_in_last_block", "int t1 = (j + 1) * P < N ? (j + 1) * P : N;",
     "int t1 = (j + 1) * P;", True),
    ("lse_without_max", "a->lse_out[(size_t)b * a->Hq + h] = m + log(den);",
     "a->lse_out[(size_t)b * a->Hq + h] = log(den);", False),
    ("values_read_from_keys", "o[d] += wt * elem(a->v_pool", "o[d] += wt * elem(a->k_pool", False),
    ("prefill_causal_off_by_one", "t <= pos;", "t < pos;", True),
    ("prefill_diagonal_not_kept", "sel[keff] = diag;", "sel[keff] = diag - 1;", False),
    ("prefill_tile_query_not_mean", "qt[d] = acc / (double)((i1 - i0) * G);",
     "qt[d] = acc / (double)G;", False),
    ("prefill_chunk_values_from_keys", "const void* src = which_v ? a->v_new : a->k_new;",
     "const void* src = a->k_new;", False),
    ("index_sum_pool_not_max", "if (s > best) best = s;", "best = (t == 0) ? s : best + s;", False),
    ("index_partial_block_reads_past_length", "int n_j = N - j * P < P ? N - j * P : P;", "int n_j = P;",
     False),
    ("index_query_of_group_zero", "elem(q_idx, dtype, ((size_t)b * Hkv + g) * Di + d)",
     "elem(q_idx, dtype, ((size_t)b * Hkv + 0) * Di + d)", False),
    ("index_key_first_token_only", "elem(ikeys, dtype, ((size_t)page * P + t) * Di + d)",
     "elem(ikeys, dtype, ((size_t)page * P + 0) * Di + d)", False),
    ("forced_local_off_by_one", "forced[j] = (char)(j < sink || j >= n - local);",
     "forced[j] = (char)(j < sink || j > n - local);", False),
    ("forced_sink_ignored", "forced[j] = (char)(j < sink || j >= n - local);",
     "forced[j] = (char)(j < 0 || j >= n - local);", False),
    ("forced_rest_in_index_order", "qsort(rest, (size_t)m, sizeof(scored_t), by_score_then_index);", "", False),
    ("decode_forced_dropped", "orc_topk_forced(s, nb, K, a->keep_sink, a->keep_local, sel)",
     "orc_topk_forced(s, nb, K, 0, 0, sel)", False),
    ("index_forced_dropped", "orc_topk_forced(row, nb, top_k, keep_sink, keep_local,",
     "orc_topk_forced(row, nb, top_k, 0, 0,", False),
    ("bf16_summary_rounding_dropped", "if (a->summary_bf16)\n        for (int d = 0; d < a->D; ++d) S[d] = round_to_bf16(S[d]);",
     "if (0)\n        for (int d = 0; d < a->D; ++d) S[d] = round_to_bf16(S[d]);", False),
    ("bf16_round_half_up", "return ldexp(rint(ldexp(m, 8)), e - 8);", "return ldexp(floor(ldexp(m, 8) + 0.5), e - 8);",
     False),
    ("bf16_truncate", "return ldexp(rint(ldexp(m, 8)), e - 8);", "return ldexp(trunc(ldexp(m, 8)), e - 8);", False),
    ("bf16_seven_bits", "return ldexp(rint(ldexp(m, 8)), e - 8);", "return ldexp(rint(ldexp(m, 7)), e - 7);", False),
    ("bf16_prefill_rounding_dropped", "        if (a->summary_bf16)\n            for",
     "        if (0)\n            for", False),
    ("prefill_forced_dropped", "orc_topk_forced(s, diag, K, a->keep_sink, a->keep_local, sel)",
     "orc_topk_forced(s, diag, K, 0, 0, sel)", False),
    # the prefill route over given lists (idx_in)
    ("prefill_idx_in_drops_diagonal", "if (sel[e] < 0 || sel[e] > diag) sel[e] = -1;",
     "if (sel[e] < 0 || sel[e] >= diag) sel[e] = -1;", False),
    ("prefill_idx_in_last_slot_dropped", "        keff = K;\n", "        keff = K - 1;\n", False),
    ("prefill_idx_in_ignored", "        memcpy(sel, a->idx_in +", "        if (0) memcpy(sel, a->idx_in +", False),
    # the index branch's rows
    ("index_scores_row_of_other_group", "double* srow = scores_out + ((size_t)b * Hkv + g) * max_blocks;",
     "double* srow = scores_out + ((size_t)b * Hkv + (Hkv - 1 - g)) * max_blocks;", False),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,orig,bad,every", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, orig, bad, every, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) >= 1, "mutation target not found: %s" % name
    mutated = src.replace(orig, bad) if every else src.replace(orig, bad, 1)
    c_file = tmp_path / "oracle_mutant.c"
    c_file.write_text(mutated)
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(c_file), "-o",
                    str(lib), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, MSA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "the pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
