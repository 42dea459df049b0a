"""The oracle's pins must be sensitive: planted mistakes must make one of them fail.

Each case copies oracle/hstu_oracle.c, plants one plausible mistake by a textual
substitution (a dropped term, a wrong sign or index, an alternative reading of
an open point of the pages), compiles the mutant with gcc into a temporary
directory, swaps it in as the oracle, and runs the pin tests.  At least one pin
must fail.  The committed oracle is never modified.
"""
import os

import pytest

import oracle
import test_oracle_mask as TM
import test_oracle_numerics as TN
import test_oracle_rab as TR

SRC = os.path.join(os.path.dirname(oracle.__file__), "hstu_oracle.c")

MUTATIONS = {
    "local_bound_strict": ("return d <= s->L && d >= -s->L;", "return d < s->L && d > -s->L;"),
    "target_key_visible": ("if (j >= s->Ck + s->Ukv) return 0;", "if (j > s->Ck + s->Ukv) return 0;"),
    "context_rows_see_uih": ("if (s->causal) return 0;         /* precedes",
                             "if (s->causal) return 1;         /* precedes"),
    "minfull_off_by_one": ("u >= s->Uq - s->M", "u > s->Uq - s->M"),
    "targets_ignore_minfull": ("full = (s->L == 0) || (s->M > 0);", "full = (s->L == 0);"),
    "cross_top_left": ("x = u + (s->Ukv - s->Uq);", "x = u;"),
    "silu_sign": ("x / (1 + R_EXP(-x))", "x / (1 + R_EXP(x))"),
    "alpha_dropped": ("sbuf[j] = al * dot +", "sbuf[j] = dot +"),
    "rab_bucket_strict": ("if (kRabEdges[e] <= d) b = e + 1;", "if (kRabEdges[e] < d) b = e + 1;"),
    "rab_time_head_zero": ("r->time_tab[(int64_t)h * RAB_BUCKETS", "r->time_tab[(int64_t)0 * RAB_BUCKETS"),
    "rab_pos_signed": ("int d = i > j ? i - j : j - i;", "int d = i > j ? i - j : 0;"),
    "rab_pos_clamp": ("imin(d, r->P - 1)", "imin(d, r->P - 2)"),
    "rab_time_gap_reversed": ("(int64_t)r->ts[s->q0 + i] - (int64_t)r->ts[s->kv0 + j]",
                              "(int64_t)r->ts[s->q0 + i] + (int64_t)r->ts[s->kv0 + j]"),
    "default_alpha": ("1.0 / sqrt((double)p->Dqk)", "1.0 / (double)p->Dqk"),
    "wrong_head_of_k": ("const float *kj = k + ((s->kv0 + j) * H + h)",
                        "const float *kj = k + ((s->kv0 + j) * H + 0)"),
    "v_row_of_query": ("const float *vj = v + ((s->kv0 + j) * H + h) * (int64_t)Dv;\n"
                       "            for (int e = 0; e < Dv; ++e) acc[e] += p * (real_t)vj[e];\n"
                       "        }\n        for",
                       "const float *vj = v + ((s->kv0 + i) * H + h) * (int64_t)Dv;\n"
                       "            for (int e = 0; e < Dv; ++e) acc[e] += p * (real_t)vj[e];\n"
                       "        }\n        for"),
    "silu_attn_scale_dropped": ("        for (int e = 0; e < Dv; ++e) o_row[e] = (double)(acc[e] * a);\n"
                                "        if (lse_out) *lse_out = 0.0;",
                                "        for (int e = 0; e < Dv; ++e) o_row[e] = (double)acc[e];\n"
                                "        if (lse_out) *lse_out = 0.0;"),
    "lse_without_max": ("real_t lse = smax + R_LOG(denom);", "real_t lse = R_LOG(denom);"),
    "softmax_unnormalised": ("real_t p = R_EXP(sbuf[j] - lse);", "real_t p = R_EXP(sbuf[j] - smax);"),
    "group_interleaved": ("return b / (p->B / p->G);", "return b % p->G;"),
    "default_scale_physical_len": ("seqs[b].Uq > mx) mx = seqs[b].Uq;",
                                   "seqs[b].S_q > mx) mx = seqs[b].S_q;"),
}


def _pins():
    """Every pin of the two oracle test modules, as zero-argument callables."""
    out = [TM.test_pair_count_readme_batched_example, TM.test_pair_count_readme_jagged_example,
           TM.test_pair_count_cross_example, TM.test_plain_causal_is_lower_triangular,
           TM.test_local_window_shape, TM.test_degenerate_lengths_are_clamped]
    for args in [(0, 9, 0, 0, 0), (3, 7, 2, 2, 0), (2, 12, 3, 3, 4), (4, 20, 5, 6, 7)]:
        out.append(lambda a=args: TM.test_mask_invariants(*a))
    out.append(TN.test_worked_example_silu_mass)
    for causal in (True, False):
        out.append(lambda c=causal: TN.test_softmax_equals_sdpa(c, 64, 64))
    out.append(TN.test_default_alpha_is_inverse_sqrt_hdim)
    out.append(lambda: TN.test_silu_equals_dense_masked_product(4, 32))
    out += [TN.test_cross_attention_bottom_right_alignment, TN.test_empty_rows,
            TN.test_group_call_equals_separate_calls,
            TN.test_attn_scale_default_is_inverse_max_uih_of_group,
            TM.test_mask_matches_enumerator_self_attention,
            TM.test_mask_matches_enumerator_cross_attention]
    out.append(TR.test_time_buckets_match_the_table)
    for causal in (True, False):
        out.append(lambda c=causal: TR.test_softmax_with_bias_equals_sdpa(c, "both"))
    out += [TR.test_silu_with_bias_equals_dense_product, TR.test_constant_positional_bias_only_shifts_softmax]
    return out


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    find, repl = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(find, repl))
    lib = oracle.load(oracle.build(src=str(mut), out=str(tmp_path / "mutant.so")))
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = None
    for pin in _pins():
        try:
            pin()
        except AssertionError as e:  # the pin noticed the planted mistake
            caught = e
            break
    assert caught is not None, f"no pin fails for the planted mistake {name}"
