"""The pins catch plausible mistakes: each case plants one mistake in a copy of
the oracle's C source (on the CPU), rebuilds it, and checks that at least one
pin fails against the planted copy."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_gate as TG
import test_oracle_indexer as TI
import test_oracle_mla as TM
import test_oracle_topk as TT
import test_oracle_write as TW

MUTANTS = {
    "dropped_relu": ("if (dot > 0.0)\n                    I +=", "if (1)\n                    I +="),
    "dropped_weight": ("I += (double)w[(int64_t)t * H_I + h] * dot;", "I += dot;"),
    "key_row_ignores_base": ("k_idx + (base[t] + s) * (int64_t)D_I", "k_idx + (int64_t)s * D_I"),
    "transposed_q": ("qd[(int64_t)h * D_I + d] * kd[d]", "qd[(int64_t)d * H_I + h % H_I] * kd[d]"),
    "ties_prefer_higher_position": ("return (a->pos > b->pos) - (a->pos < b->pos);",
                                    "return (a->pos < b->pos) - (a->pos > b->pos);"),
    "ascending_scores": ("if (a->score > b->score) return -1;\n    if (a->score < b->score) return 1;",
                         "if (a->score < b->score) return -1;\n    if (a->score > b->score) return 1;"),
    "sink_missing_from_denominator": ("double den = exp((double)sink[h] - m);", "double den = 0.0;"),
    "sink_carries_value": ("o[v] /= den;", "o[v] = (o[v] + exp((double)sink[h] - m)) / den;"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "value_from_trailing_dims": ("o[v] += p * orc_bf16_to_double(kr[v]);",
                                 "o[v] += p * orc_bf16_to_double(kr[D_qk - D_v + v]);"),
    "fp8_wrong_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "fp8_no_subnormal": ("v = ldexp((double)m / 8.0, -6);", "v = 0.0;"),
    "padding_not_skipped": ("if (row[j] < 0)\n                    continue;\n                const uint16_t *kr = kv + (base[t] + row[j]) * (int64_t)D_qk;\n                double p",
                            "if (row[j] < -1)\n                    continue;\n                const uint16_t *kr = kv + (base[t] + (row[j] < 0 ? 0 : row[j])) * (int64_t)D_qk;\n                double p"),
    "gate_sign_flipped": ("acc / (1.0 + exp(-g))", "acc / (1.0 + exp(g))"),
    "gate_dropped": ("= acc / (1.0 + exp(-g));", "= acc;"),
    "wv_b_transposed": ("acc += orc_bf16_to_double(wr[c]) * orc_bf16_to_double(ot[c]);",
                        "acc += orc_bf16_to_double(wv_b[((int64_t)h * D_v + c) * D_o + e]) * orc_bf16_to_double(ot[c]);"),
    "gate_in_latent_space": ("const double g = orc_bf16_to_double(gate[((int64_t)t * H + h) * D_o + e]);",
                             "const double g = orc_bf16_to_double(gate[((int64_t)t * H + h) * D_o + (e % 2) * 4 + 1]);"),
    "rope_neox_pairs": ("const double x0 = x[2 * i], x1 = x[2 * i + 1];\n        x[2 * i] = x0 * c - x1 * s;\n        x[2 * i + 1] = x1 * c + x0 * s;",
                        "const double x0 = x[i], x1 = x[i + D_rope / 2];\n        x[i] = x0 * c - x1 * s;\n        x[i + D_rope / 2] = x1 * c + x0 * s;"),
    "rope_sign_flipped": ("x[2 * i] = x0 * c - x1 * s;", "x[2 * i] = x0 * c + x1 * s;"),
    "rope_sin_cos_swapped": ("const double c = cs[i], s = cs[D_rope / 2 + i];", "const double s = cs[i], c = cs[D_rope / 2 + i];"),
    "ln_unbiased_variance": ("var /= D_I;", "var /= (D_I - 1);"),
    "ln_bias_dropped": (" * (double)ln_w[d] + (double)ln_b[d];", " * (double)ln_w[d];"),
    "ln_eps_outside_sqrt": ("1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    "key_rope_on_leading_span": ("orc_rope_interleaved(yt + (D_I - D_rope), D_rope, rope, pos[t]);",
                                 "orc_rope_interleaved(yt, D_rope, rope, pos[t]);"),
    "latent_rope_on_leading_span": ("orc_rope_interleaved(ot + (D_qk - D_rope), D_rope, rope, pos[t]);",
                                    "orc_rope_interleaved(ot, D_rope, rope, pos[t]);"),
    "fp8_ties_away_from_zero": ("if (d < bd || (d == bd && (c & 1) == 0)) {", "if (d <= bd) {"),
    "fp8_truncates": ("const double d = fabs(orc_fp8_e4m3fn_to_double((uint8_t)c) - a);",
                      "const double d = orc_fp8_e4m3fn_to_double((uint8_t)c) <= a ? a - orc_fp8_e4m3fn_to_double((uint8_t)c) : INFINITY;"),
}


def run_pins():
    """Run every pin; return the names of those that fail."""
    failed = []
    cases = [
        ("fp8", lambda: __import__("test_oracle_decoders").test_fp8_e4m3fn_all_codes(oracle)),
        ("idx_einsum", lambda: TI.test_against_int64_einsum(oracle, "tiny_2layer")),
        ("idx_const", lambda: [TI.test_closed_form_constant(oracle, c) for c in (-3.0, 2.0, 0.5)]),
        ("idx_signed", lambda: TI.test_closed_form_signed_heads(oracle)),
        ("idx_rows", lambda: TI.test_rows_follow_base_and_length(oracle)),
        ("topk_ties", lambda: TT.test_brute_force_ties(oracle, 0)),
        ("topk_real", lambda: TT.test_brute_force_real_values(oracle, 0)),
        ("mla_dense", lambda: TM.test_dense_equals_torch_sink_softmax(oracle, 0)),
        ("mla_zero_q", lambda: TM.test_zero_query_is_mean_with_sink(oracle)),
        ("mla_single", lambda: TM.test_single_key_is_sigmoid(oracle)),
        ("mla_perm", lambda: TM.test_permutation_and_padding_invariant(oracle)),
        ("mla_value", lambda: TM.test_value_is_leading_part_and_linear(oracle)),
        ("mla_base", lambda: TM.test_rows_offset_by_base(oracle)),
        ("gate_identity", lambda: TG.test_identity_upprojection(oracle)),
        ("gate_rank1", lambda: TG.test_rank1_closed_form(oracle)),
        ("gate_logistic", lambda: TG.test_gate_is_logistic(oracle)),
        ("gate_heads", lambda: TG.test_heads_permute(oracle)),
        ("fp8_codes", lambda: TW.test_fp8_every_code_round_trips(oracle)),
        ("fp8_mid", lambda: TW.test_fp8_midpoints_tie_to_even(oracle)),
        ("fp8_torch", lambda: TW.test_fp8_matches_torch_cast_in_range(oracle)),
        ("fp8_sat", lambda: TW.test_fp8_saturates(oracle)),
        ("ln_torch", lambda: TW.test_layer_norm_matches_torch(oracle, 64)),
        ("ln_const", lambda: TW.test_layer_norm_constant_row_gives_bias(oracle)),
        ("rope_latent", lambda: TW.test_latent_row_rotates_trailing_pairs(oracle)),
        ("rope_relpos", lambda: TW.test_rope_relative_position(oracle)),
        ("rope_key", lambda: TW.test_index_key_rotates_trailing_span(oracle)),
    ]
    for name, fn in cases:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_unmutated_oracle_passes_every_pin(orc):
    assert run_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(orc, mutant_dir, name):
    before, after = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(before) == 1, name
    path = os.path.join(str(mutant_dir), f"{name}.c")
    so = os.path.join(str(mutant_dir), f"{name}.so")
    open(path, "w").write(src.replace(before, after))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", path, "-o", so, "-lm"])
    saved_lib, saved_path = oracle._lib, oracle._LIB
    try:
        oracle._lib, oracle._LIB = None, so
        oracle.lib()
        failed = run_pins()
    finally:
        oracle._lib, oracle._LIB = saved_lib, saved_path
    assert failed, f"no pin caught mutant {name}"
