"""The oracle's pins must be able to fail.

Each case below plants one plausible mistake in a copy of oracle.c (a dropped
term, float accumulation, a transposed operand, a wrong e4m3 bias or sign,
rounding twice, the wrong tie rule, a lost scale, a lost subnormal clamp, an
ignored row stride; for MXFP8: the wrong block size or block index, the wrong
scale bias, swapped scale arrays, a NaN scale read as finite, an ignored scale
stride; for attention: a dropped scale, a causal mask that is off by one or
missing, the wrong grouped-query head, no max shift, no log in the LSE, keys
read as values, a dropped last key, rounding through float, an ignored head
stride, a tolerance magnitude that is not normalised or not taken of |v|),
builds the copy on the CPU in a temporary directory, and
runs the pins of test_oracle.py, test_oracle_mx.py and test_oracle_attn.py
against it.  At least one pin must fail for
every mutant.  The oracle itself is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_attn as attn_pins
from tests import test_oracle_mx as mx_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dropped_last_term": ("for (k = 0; k < K; ++k)", "for (k = 0; k + 1 < K; ++k)"),
    "float_accumulation": ("double acc = 0.0, mag = 0.0;", "float acc = 0.0f; double mag = 0.0;"),
    "transposed_B": ("B, j * ldb + k", "B, k * ldb + j"),
    "ignored_lda": ("A, i * lda + k", "A, i * K + k"),
    "e4m3_bias_8": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_no_sign": ("return s ? -mag : mag;", "return mag;"),
    "e4m3_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "double_rounding": ("r = rint(ax / q) * q;", "r = rint((double)(float)ax / q) * q;"),
    "ties_away": ("r = rint(ax / q) * q;", "r = round(ax / q) * q;"),
    "lost_scale": ("*c_out = acc * s;", "*c_out = acc;"),
    "no_subnormal_clamp": ("E = -126;", "E = E;"),
    "mx_block_of_16": ("k / 32]", "k / 16]"),
    "mx_block_off_by_one": ("SA[i * ldsa + k / 32]", "SA[i * ldsa + (k + 1) / 32]"),
    "mx_scale_bias_128": ("ldexp(1.0, (int)x - 127)", "ldexp(1.0, (int)x - 128)"),
    "mx_scales_swapped": ("xtab[SA[i * ldsa + k / 32]]", "xtab[SB[i * ldsb + k / 32]]"),
    "mx_nan_scale_ignored": ("if (x == 255)\n        return NAN;", "if (x == 255)\n        return 1.0;"),
    "mx_ignored_ldsa": ("SA[i * ldsa + k / 32]", "SA[i * ((K + 31) / 32) + k / 32]"),
    "attn_no_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "attn_causal_strict": ("causal ? i + 1 : N", "causal ? i : N"),
    "attn_causal_ignored": ("causal ? i + 1 : N", "N"),
    "attn_gqa_modulo": ("h / (Hq / Hkv)", "h % Hkv"),
    "attn_no_max_shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "attn_lse_no_log": ("*lse = m + log(l);", "*lse = m + l;"),
    "attn_keys_as_values": ("V[b * sv[0] + kvh * sv[1] + j * sv[2] + d]",
                            "K[b * sk[0] + kvh * sk[1] + j * sk[2] + d]"),
    "attn_dropped_last_key": ("for (j = 0; j < nk; ++j) {\n            const double v",
                              "for (j = 0; j + 1 < nk; ++j) {\n            const double v"),
    "attn_rounded_through_float": ("o[d] = oracle_bf16_round(val);",
                                   "o[d] = oracle_bf16_round((double)(float)val);"),
    "attn_ignored_head_stride": ("h * sq[1]", "h * D"),
    "attn_amag_unnormalised": ("amag[d] = mag / l;", "amag[d] = mag;"),
    "attn_amag_signed": ("mag += s[j] * fabs(v);", "mag += s[j] * v;"),
}

PINS = [
    lambda m: [pins.test_golden_fixture(m, c) for c in pins.GOLDEN_CASES],
    pins.test_e4m3_table_matches_torch,
    pins.test_e4m3_landmarks,
    pins.test_bf16_round_single_rounding_cases,
    pins.test_bf16_round_matches_torch_ties_and_edges,
    lambda m: pins.test_integer_bf16_exact(m, 17, 9, 33, 3),
    lambda m: pins.test_integer_fp8_exact_with_power_of_two_scales(m, 4, 4, 16),
    lambda m: pins.test_fraction_bruteforce_bf16(m, 0),
    lambda m: pins.test_fraction_bruteforce_fp8(m, 0),
    pins.test_identity_B_bf16,
    pins.test_non_square_orientation,
    pins.test_strided_equals_packed,
    mx_pins.test_unit_scales_equal_plain_fp8,
    lambda m: mx_pins.test_fraction_bruteforce(m, 0),
    mx_pins.test_integer_valued_against_torch_matmul,
    mx_pins.test_block_boundaries,
    mx_pins.test_nan_scale_poisons_its_row_only,
    mx_pins.test_strided_equals_packed,
    lambda m: attn_pins.test_matches_torch_sdpa_float64(m, 2, 4, 2, 7, 8, False),
    lambda m: attn_pins.test_matches_torch_sdpa_float64(m, 2, 4, 2, 7, 8, True),
    lambda m: attn_pins.test_correctly_rounded_against_mpmath(m, 0, True),
    lambda m: attn_pins.test_zero_queries_give_the_mean_of_visible_values(m, True),
    attn_pins.test_mean_that_double_rounding_gets_wrong,
    attn_pins.test_single_key_returns_its_value_row,
    attn_pins.test_first_causal_row_sees_only_key_zero,
    attn_pins.test_dominant_key_gives_its_value_row,
    attn_pins.test_grouped_query_heads_equal_repeated_heads,
    attn_pins.test_strided_equals_packed,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, monkeypatch, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor missing: %r" % old
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(text.replace(old, new))
    lib_path = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-ffp-contract=off", "-o", str(lib_path), str(mutant_src), "-lm"],
                   check=True)
    monkeypatch.setattr(oracle, "_LIB", str(lib_path))
    monkeypatch.setattr(oracle, "_lib", None)
    oracle._load()
    failed = []
    for pin in PINS:
        try:
            pin(oracle)
        except (AssertionError, ValueError) as e:  # a pin fired
            failed.append(getattr(pin, "__name__", "pin"))
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, "no pin caught mutant %s" % name
