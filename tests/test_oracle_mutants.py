"""Planted mistakes in the oracle (CPU only): each mutant copy of oracle.c must
fail at least one pin, which shows the pins constrain the arithmetic they cover."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "no_relu": ("if (dot > 0) s += (int64_t)w[h] * dot;", "s += (int64_t)w[h] * dot;",
                [pins.test_scores_sign_symmetry]),
    "head_weight_index": ("s += (int64_t)w[h] * dot", "s += (int64_t)w[31 - h] * dot",
                          [lambda rng: pins.test_scores_one_hot_weight_is_relu_of_gemv(rng, 1)]),
    "transposed_query": ("(int64_t)q[h * OR_IDX_DIM + d]", "(int64_t)q[d * OR_IDX_HEADS + h]",
                         [lambda rng: pins.test_scores_one_hot_weight_is_relu_of_gemv(rng, 17)]),
    "tail_not_renormalised": ("if (r == OR_GROUP) return acc;", "return acc;",
                              [pins.test_pool_impulse_response_places_each_weight]),
    "pool_plain_mean": ("acc += w[i] * bf16_value", "acc += 0.25 * bf16_value",
                        [pins.test_pool_impulse_response_places_each_weight]),
    "pool_weights_reversed": ("acc += w[i] * bf16_value", "acc += w[3 - i] * bf16_value",
                              [pins.test_pool_impulse_response_places_each_weight]),
    "amax_without_abs": ("if (fabs(v) > amax) amax = fabs(v);", "if (v > amax) amax = v;",
                         [lambda rng: pins.test_quantisation_properties(0),
                          lambda rng: pins.test_quantisation_properties(1)]),
    "round_half_away": ("nearbyint(x / scale)", "round(x / scale)",
                        [lambda rng: pins.test_quantisation_round_half_even()]),
    "ties_prefer_high_index": ("return (x->group > y->group) - (x->group < y->group);",
                               "return (x->group < y->group) - (x->group > y->group);",
                               [pins.test_topk_ties_straddling_the_threshold]),
    "ascending_scores": ("return x->score > y->score ? -1 : 1;", "return x->score > y->score ? 1 : -1;",
                         [lambda rng: pins.test_topk_matches_rank_count_brute_force(rng, 1000, 1_000_000)]),
    "prefill_mask_off_by_one": ("S[g] = g <= last ?", "S[g] = g < last ?",
                                [lambda rng: pins.test_prefill_block_causal_mask(rng, 7)]),
    "causal_off_by_one": ("if (t < L && t <= pos)", "if (t < L && t < pos)",
                          [pins.test_attention_single_token_returns_that_row]),
    "missing_softmax_scale": ("s[i] = dot * scale;", "s[i] = dot;",
                              [lambda rng: pins.test_attention_dense_fallback_is_textbook_attention(rng, 100)]),
    "reads_past_sequence_end": ("if (t < L && t <= pos)", "if (t <= pos)",
                                [pins.test_attention_order_invariance_and_causality]),
    "fp8_bias_8": ("v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 11);",
                   [lambda rng: pins.test_fp8_decode_table()]),
    "fp8_ties_away": ("double q = nearbyint(ldexp(a, 3 - ub));", "double q = round(ldexp(a, 3 - ub));",
                      [lambda rng: pins.test_fp8_encode_round_trip_and_nearest()]),
    "fp8_scale_int8_range": ("float s = amax > 0.f ? amax / 448.f : 1.f;", "float s = amax > 0.f ? amax / 127.f : 1.f;",
                             [pins.test_latent_fp8_rows]),
    "kda_decay_dropped": ("Sp[i * D + j] = (double)alpha[i] * bf16_value(S[i * D + j]);",
                          "Sp[i * D + j] = bf16_value(S[i * D + j]);", [pins.test_kda_decay_scales_key_rows]),
    "kda_erase_sign": ("(bf16_value(v[j]) - u)", "(bf16_value(v[j]) + u)",
                       [pins.test_kda_delta_rule_is_the_pages_equation]),
    "kda_readout_transposed": ("acc += bf16_value(q[i]) * Sp[i * D + j];", "acc += bf16_value(q[i]) * Sp[j * D + i];",
                               [pins.test_kda_no_erase_no_decay_keeps_state]),
    "kda_readout_of_old_state": ("acc += bf16_value(q[i]) * Sp[i * D + j];", "acc += bf16_value(q[i]) * bf16_value(S[i * D + j]);",
                                 [pins.test_kda_writes_the_value_at_a_unit_key]),
    "fp8_row_scale_ignored": ("return (double)c->scales[t] * oracle_fp8_decode", "return oracle_fp8_decode",
                              [pins.test_attention_fp8_equals_bf16_attention_on_exact_values]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    old, new, checks = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(SRC), "oracle.h")
    (tmp_path / "oracle.h").write_text(open(hdr).read())
    so = str(tmp_path / "liboracle_mut.so")
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(mut), "-o", so, "-lm"])
    caught = False
    with oracle.use_library(so):
        for chk in checks:
            try:
                chk(np.random.default_rng(7))
            except AssertionError:
                caught = True
                break
    assert caught, f"no pin caught the planted mistake '{name}'"
