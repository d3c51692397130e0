"""Mutation check of the oracle pins: each case compiles a copy of the oracle
with one plausible mistake planted (on the CPU, in a temporary directory) and
requires that at least one of the named pins rejects it."""
import os
import sys

import pytest

import oracle

sys.path.insert(0, os.path.dirname(__file__))
import test_oracle_gemm as tg      # noqa: E402
import test_oracle_mxfp4 as t4     # noqa: E402
import test_oracle_mxfp4_gemm as t4g  # noqa: E402
import test_oracle_mxfp8 as t8     # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "mxq_oracle.c")

MUTANTS = {
    "fp4 ties round down": ("if (yabs >= fp4_midpoints[i]) idx = i + 1;",
                            "if (yabs > fp4_midpoints[i]) idx = i + 1;",
                            [lambda: t4.test_midpoint_ties_go_to_larger_magnitude(0)]),
    "fp4 exponent floor instead of round": (
        "while (a2 >= s2 * ldexp(2.0, 2 * n)) n++;\n    while (a2 < s2 * ldexp(0.5, 2 * n)) n--;",
        "while (a2 >= s2 * ldexp(4.0, 2 * n)) n++;\n    while (a2 < s2 * ldexp(1.0, 2 * n)) n--;",
                               [t4.test_exponent_round_half_threshold]),
    "fp4 saturation mask uses >=": ("if (fabs(v[i]) > FP4_CODE_MAX * scale) *byte |= bit;",
                                    "if (fabs(v[i]) >= FP4_CODE_MAX * scale) *byte |= bit;",
                                    [t4.test_saturation_mask_marks_values_beyond_six_scales]),
    "fp4 scale factor ignored": ("int e = fp4_scale_exp(amax, scale_factor);",
                                 "int e = fp4_scale_exp(amax, 6.0);",
                                 [t4.test_scale_factor_threshold_for_several_factors]),
    "fp4 ste mask row stride": ("int sat = (sat_mask[r * (Lp / 8) + c / 8] >> (c % 8)) & 1;",
                                "int sat = (sat_mask[r * (L / 8) + c / 8] >> (c % 8)) & 1;",
                                [t4.test_ste_backward_zeroes_only_clipped_elements]),
    "fp4 dequant nibble order": ("uint8_t nib = (c % 2 == 0) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4);",
                                 "uint8_t nib = (c % 2 == 1) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4);",
                                 [lambda: t4g.test_dequant_reproduces_qdq_output((3, 17), 6.0)]),
    "fp4 decode exponent bias": ("(1.0 + 0.5 * m) * ldexp(1.0, e - 1);", "(1.0 + 0.5 * m) * ldexp(1.0, e - 2);",
                                 [t4g.test_dequant_of_every_nibble_is_the_page_codebook]),
    "fp4 gemm operand rows shifted": ("double p = Xa[m * K + k] * Xb[n * K + k];",
                                      "double p = Xa[m * K + k] * Xb[((n + 1) % N) * K + k];",
                                      [t4g.test_gemm_fp4_equals_matmul_of_qdq_outputs]),
    "fp4 min scale 2^-31": ("#define FP4_MIN_SCALE_EXP (-30)", "#define FP4_MIN_SCALE_EXP (-31)",
                            [t4.test_zero_and_tiny_blocks_use_minimum_scale]),
    "fp4 drops sign of zero": ("double out = copysign(fp4_codebook[idx] * scale, v[i]);",
                               "double out = (v[i] < 0 ? -1.0 : 1.0) * fp4_codebook[idx] * scale;",
                               [t4.test_zero_and_tiny_blocks_use_minimum_scale]),
    "fp4 flattens before padding": ("v[i] = col < L ? (double)x[r * L + col] : 0.0;",
                                    "v[i] = col < L ? (double)x[r * L + col] : (r + 1 < rows ? (double)x[(r + 1) * L + col - L] : 0.0);",
                                    [t4.test_rows_are_padded_separately]),
    "e4m3 ties away from zero": ("else code = (uint8_t)((lo & 1) == 0 ? lo : hi);",
                                 "else code = (uint8_t)hi;",
                                 [t8.test_e4m3_encode_every_distinct_input_matches_torch]),
    "mxfp8 emax 7": ("int s = (e2 - 1) - 8;", "int s = (e2 - 1) - 7;",
                     [t8.test_scale_byte_is_exponent_field_minus_8]),
    "grouped blocks do not restart": ("P += ceil32(m);\n            start = end;",
                                      "P += m;\n            start = end;",
                                      [lambda: t8.test_grouped_colT_is_per_group_colT([0, 1, 31, 32, 33, 0])]),
    "gemm reverses K of B": ("double p = Ad[m * K + k] * Bd[n * K + k];",
                             "double p = Ad[m * K + k] * Bd[n * K + (K - 1 - k)];",
                             [lambda: tg.test_gemm_equals_numpy_matmul_of_dequantised(17, 9, 96)]),
    "ragged-k sums only the first group": ("dot_range(A, sA, m, B, sB, n, ldk, P[g], P[g + 1], &C[o], &Cabs[o]);",
                                           "dot_range(A, sA, m, B, sB, n, ldk, P[0], P[1], &C[o], &Cabs[o]);",
                                           [lambda: tg.test_ragged_k_is_dense_per_group_and_empty_is_zero([5, 0, 33, 1, 40])]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new, pins = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    caught = 0
    with oracle.using(lib):
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError):
                caught += 1
    assert caught, f"no pin caught the planted mistake '{name}'"
