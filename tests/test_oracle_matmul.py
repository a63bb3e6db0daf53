"""Pins for the oracle's matmul path (oracle/matmul.py).  CPU only.

The matmul path computes the same product as the loop oracle with the double
sum taken by numpy's matrix product; it is what lets the GPU tests compare
full-size outputs element by element.  It is pinned here three ways:

* every pin of test_oracle.py, test_oracle_mx.py and test_oracle_attn.py
  that calls the product or the attention forward (hand-derived fixtures,
  exact rationals, integer-valued products against int64 and torch,
  identities, strides, NaN scales; torch's float64 SDPA, mpmath, closed forms,
  invariants) runs against it, with the rows taken in chunks of 5 so the chunk
  loop is exercised;
* on random operands with padded strides it agrees with the loop oracle bit
  for bit in C (and O) and to a few double roundings in S (and LSE, A);
* planted mistakes in a copy of its source each make at least one of those
  pins fail.
"""
import importlib.util

import numpy as np
import pytest

import oracle
from oracle import matmul
from tests import test_oracle as pins
from tests import test_oracle_attn as attn_pins
from tests import test_oracle_mx as mx_pins


class MatmulOracle:
    """The oracle package with gemm and gemm_mx taken by a matmul-path module."""

    def __init__(self, mod, rows_per_chunk=5):
        self._mod = mod
        self._rpc = rows_per_chunk

    def __getattr__(self, name):
        return getattr(oracle, name)

    def gemm(self, dtype, A, B, M, N, K, lda=None, ldb=None, scale_a=1.0, scale_b=1.0,
             threads=None, want_s=True):
        return self._mod.gemm_by_matmul(dtype, A, B, M, N, K, lda, ldb, scale_a, scale_b,
                                        want_s, self._rpc)

    def gemm_mx(self, A, B, SA, SB, M, N, K, lda=None, ldb=None, ldsa=None, ldsb=None,
                threads=None, want_s=True):
        return self._mod.gemm_mx_by_matmul(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb,
                                           want_s, self._rpc)

    def attention(self, Q, K, V, B, Hq, Hkv, N, D, scale, causal, q_strides=None,
                  k_strides=None, v_strides=None, rows=None, threads=None):
        return self._mod.attention_by_matmul(Q, K, V, B, Hq, Hkv, N, D, scale, causal, q_strides,
                                             k_strides, v_strides, rows, self._rpc)


PINS = {
    "golden_fixtures": lambda m: [pins.test_golden_fixture(m, c) for c in pins.GOLDEN_CASES],
    "integer_bf16": lambda m: [pins.test_integer_bf16_exact(m, *p) for p in
                               [(1, 1, 1, 0), (3, 5, 7, 0), (17, 9, 33, 3), (64, 48, 200, 8),
                                (5, 70, 1024, 0)]],
    "integer_fp8": lambda m: [pins.test_integer_fp8_exact_with_power_of_two_scales(m, *p)
                              for p in [(4, 4, 16), (33, 17, 300), (8, 64, 1000)]],
    "integer_workload_generator": pins.test_integer_from_the_workload_generator,
    "fraction_bf16": lambda m: [pins.test_fraction_bruteforce_bf16(m, s) for s in range(6)],
    "fraction_ties": pins.test_fraction_bruteforce_ties,
    "fraction_fp8": lambda m: [pins.test_fraction_bruteforce_fp8(m, s) for s in range(4)],
    "identity_bf16": pins.test_identity_B_bf16,
    "identity_fp8": pins.test_identity_B_fp8_power_of_two_scales,
    "transpose_identity": pins.test_transpose_identity_all_tiny_shapes,
    "non_square_orientation": pins.test_non_square_orientation,
    "strided_equals_packed": pins.test_strided_equals_packed,
    "sampled_loop_equals_full": pins.test_sampled_equals_full,
    "zero_k": pins.test_zero_k_gives_plus_zero,
    "mx_unit_scales": mx_pins.test_unit_scales_equal_plain_fp8,
    "mx_fraction": lambda m: [mx_pins.test_fraction_bruteforce(m, s) for s in range(4)],
    "mx_integer_torch": mx_pins.test_integer_valued_against_torch_matmul,
    "mx_block_boundaries": mx_pins.test_block_boundaries,
    "mx_nan_scale": mx_pins.test_nan_scale_poisons_its_row_only,
    "mx_strided_equals_packed": mx_pins.test_strided_equals_packed,
    "mx_sampled_loop_equals_full": mx_pins.test_sampled_equals_full,
    "attn_torch_sdpa": lambda m: [attn_pins.test_matches_torch_sdpa_float64(m, *p, c) for p in
                                  [(1, 1, 1, 1, 8), (2, 4, 2, 7, 8), (1, 2, 1, 33, 64),
                                   (1, 3, 3, 20, 16)] for c in (False, True)],
    "attn_mpmath": lambda m: [attn_pins.test_correctly_rounded_against_mpmath(m, s, c)
                              for s in range(3) for c in (False, True)],
    "attn_zero_queries": lambda m: [attn_pins.test_zero_queries_give_the_mean_of_visible_values(m, c)
                                    for c in (False, True)],
    "attn_single_rounding": attn_pins.test_mean_that_double_rounding_gets_wrong,
    "attn_single_key": attn_pins.test_single_key_returns_its_value_row,
    "attn_first_causal_row": attn_pins.test_first_causal_row_sees_only_key_zero,
    "attn_dominant_key": attn_pins.test_dominant_key_gives_its_value_row,
    "attn_grouped_heads": attn_pins.test_grouped_query_heads_equal_repeated_heads,
    "attn_scale_two": attn_pins.test_scale_two_equals_doubled_queries,
    "attn_strided": attn_pins.test_strided_equals_packed,
    "attn_rows_subset": attn_pins.test_rows_subset_equals_full,
    "attn_rejects": attn_pins.test_rejects_bad_arguments,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_matmul_path_passes_the_oracle_pins(name):
    PINS[name](MatmulOracle(matmul))


def _random_bf16(rng, rows, ld):
    return pins._torch_bf16_bits(rng.standard_normal(rows * ld).astype(np.float32))


@pytest.mark.parametrize("M,N,K,pad_a,pad_b,chunk", [(67, 53, 1000, 8, 3, 16), (1, 1, 1, 0, 0, 1),
                                                     (130, 7, 333, 1, 0, 1024)])
def test_bf16_agrees_with_the_loop(M, N, K, pad_a, pad_b, chunk):
    rng = np.random.default_rng(M + N + K)
    A = _random_bf16(rng, M, K + pad_a)
    B = _random_bf16(rng, N, K + pad_b)
    C0, S0 = oracle.gemm("bf16", A, B, M, N, K, lda=K + pad_a, ldb=K + pad_b)
    C1, S1 = matmul.gemm_by_matmul("bf16", A, B, M, N, K, K + pad_a, K + pad_b,
                                   rows_per_chunk=chunk)
    assert np.array_equal(C0, C1)
    assert np.allclose(S0, S1, rtol=K * 2.0 ** -52, atol=0)


def test_fp8_agrees_with_the_loop():
    rng = np.random.default_rng(2)
    tab = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    M, N, K, ld = 45, 61, 777, 800
    A = rng.choice(codes, M * ld)
    B = rng.choice(codes, N * ld)
    sa, sb = float(np.float32(0.37)), float(np.float32(-3.1))
    C0, S0 = oracle.gemm("fp8", A, B, M, N, K, lda=ld, ldb=ld, scale_a=sa, scale_b=sb)
    C1, S1 = matmul.gemm_by_matmul("fp8", A, B, M, N, K, ld, ld, sa, sb, rows_per_chunk=10)
    assert np.array_equal(C0, C1)
    assert np.allclose(S0, S1, rtol=K * 2.0 ** -52, atol=0)


def test_mx_agrees_with_the_loop():
    rng = np.random.default_rng(3)
    codes = mx_pins._finite_codes()
    M, N, K = 37, 29, 300
    nb = (K + 31) // 32
    A = rng.choice(codes, M * K)
    B = rng.choice(codes, N * K)
    SA = rng.integers(100, 150, M * (nb + 2)).astype(np.uint8)
    SB = rng.integers(100, 150, N * nb).astype(np.uint8)
    C0, S0 = oracle.gemm_mx(A, B, SA, SB, M, N, K, ldsa=nb + 2)
    C1, S1 = matmul.gemm_mx_by_matmul(A, B, SA, SB, M, N, K, ldsa=nb + 2, rows_per_chunk=8)
    assert np.array_equal(C0, C1)
    assert np.allclose(S0, S1, rtol=K * 2.0 ** -52, atol=0)


@pytest.mark.parametrize("B,Hq,Hkv,N,D,causal,chunk", [(2, 4, 2, 37, 64, True, 8),
                                                      (1, 3, 1, 50, 128, False, 16),
                                                      (1, 1, 1, 1, 8, True, 512),
                                                      (2, 2, 2, 129, 32, True, 128)])
def test_attention_agrees_with_the_loop(B, Hq, Hkv, N, D, causal, chunk):
    q = attn_pins._bf16((B, Hq, N, D), 5 + N, 2.0)
    k = attn_pins._bf16((B, Hkv, N, D), 6 + N, 2.0)
    v = attn_pins._bf16((B, Hkv, N, D), 7 + N)
    args = (attn_pins._bits(q).ravel(), attn_pins._bits(k).ravel(), attn_pins._bits(v).ravel(),
            B, Hq, Hkv, N, D, 0.7, causal)
    o0, v0, l0, a0 = oracle.attention(*args)
    o1, v1, l1, a1 = matmul.attention_by_matmul(*args, rows_per_chunk=chunk)
    assert np.array_equal(o0, o1)
    assert np.allclose(v1, v0, rtol=1e-13, atol=1e-13 * np.abs(a0).max())
    assert np.allclose(l1, l0, rtol=1e-14, atol=1e-14)
    assert np.allclose(a1, a0, rtol=1e-13, atol=0)


def test_rejects_short_operands():
    A = np.zeros(16, dtype=np.uint16)
    with pytest.raises(ValueError):
        matmul.gemm_by_matmul("bf16", A, A, 2, 2, 4, lda=13)
    with pytest.raises(ValueError):
        matmul.gemm_by_matmul("bf16", A, A, 2, 2, 4, lda=3)


MUTANTS = {
    "transposed_B": ("C[r0:r1] = oracle.bf16_round(((a @ b.T) + 0.0) * s)",
                     "C[r0:r1] = oracle.bf16_round(((a @ b) + 0.0) * s)"),
    "lost_scale": ("((a @ b.T) + 0.0) * s)", "((a @ b.T) + 0.0))"),
    "signed_magnitude": ("S[r0:r1] = (np.abs(a) @ b_abs.T) * abs(s)",
                         "S[r0:r1] = (a @ b.T) * abs(s)"),
    "ignored_row_stride": ("v = _rows(flat[r0 * ld:], r1 - r0, K, ld)",
                           "v = _rows(flat[r0 * K:], r1 - r0, K, K)"),
    "rounded_through_float": ("oracle.bf16_round(((a @ b.T) + 0.0) * s)",
                              "oracle.bf16_round((((a @ b.T) + 0.0) * s).astype(np.float32))"),
    "chunk_off_by_one": ("r1 = min(r0 + rows_per_chunk, M)\n        a = _decode(code",
                         "r1 = min(r0 + rows_per_chunk - 1, M)\n        a = _decode(code"),
    "bf16_read_as_fp16": ("return oracle.bf16_to_f64(v)\n    return tab[v]",
                          "return v.view(np.float16).astype(np.float64)\n    return tab[v]"),
    "attn_bf16_read_as_fp16": ("writeable=False)\n    return oracle.bf16_to_f64(v)",
                               "writeable=False)\n    return v.view(np.float16).astype(np.float64)"),
    "mx_block_of_16": ("np.repeat(x, 32, axis=1)", "np.repeat(x, 16, axis=1)"),
    "mx_scales_swapped": ("a = _decode_mx(A, SA, r0, r1, K, lda, ldsa, tab, xtab)",
                          "a = _decode_mx(A, SB, r0, r1, K, lda, ldsb, tab, xtab)"),
    "mx_scale_ignored": ("return v * np.repeat(x, 32, axis=1)[:, :K]", "return v"),
    "mx_negated": ("C[r0:r1] = oracle.bf16_round((a @ b.T) + 0.0)",
                              "C[r0:r1] = oracle.bf16_round(-(a @ b.T))"),
    "attn_no_scale": ("s = (q[i0:i1] @ k[:nk].T) * scale", "s = q[i0:i1] @ k[:nk].T"),
    "attn_causal_strict": ("s[keys[None, :nk] > np.arange(i0, i1)[:, None]] = -np.inf",
                           "s[keys[None, :nk] >= np.arange(i0, i1)[:, None]] = -np.inf"),
    "attn_causal_block_short": ("nk = i1 if causal else N", "nk = i1 - 1 if causal else N"),
    "attn_causal_ignored": ("if causal:\n                        s[keys",
                            "if False:\n                        s[keys"),
    "attn_causal_chunk_relative": ("np.arange(i0, i1)[:, None]] = -np.inf",
                                   "np.arange(0, i1 - i0)[:, None]] = -np.inf"),
    "attn_gqa_modulo": ("for h in range(kvh * group, (kvh + 1) * group):",
                        "for h in range(kvh, Hq, Hkv):"),
    "attn_no_max_shift": ("p = np.exp(s - m[:, None])", "p = np.exp(s)"),
    "attn_lse_no_log": ("lse[base + i0:base + i1] = m + np.log(l)",
                        "lse[base + i0:base + i1] = m + l"),
    "attn_keys_as_values": ("val = (p @ v[:nk]) / l[:, None]", "val = (p @ k[:nk]) / l[:, None]"),
    "attn_unnormalised": ("val = (p @ v[:nk]) / l[:, None]", "val = p @ v[:nk]"),
    "attn_amag_unnormalised": ("amag[base + i0:base + i1] = (p @ v_abs[:nk]) / l[:, None]",
                               "amag[base + i0:base + i1] = p @ v_abs[:nk]"),
    "attn_amag_signed": ("amag[base + i0:base + i1] = (p @ v_abs[:nk]) / l[:, None]",
                         "amag[base + i0:base + i1] = (p @ v[:nk]) / l[:, None]"),
    "attn_ignored_head_stride": ("off = int(b * s[0] + h * s[1])", "off = int(b * s[0] + h * N * D)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_matmul_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(matmul.__file__).read()
    assert text.count(old) == 1, "mutation anchor missing or ambiguous: %r" % old
    path = tmp_path / "matmul_mutant.py"
    path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location("matmul_mutant_" + name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    proxy = MatmulOracle(mod)
    failed = []
    for pin_name, pin in PINS.items():
        try:
            with np.errstate(all="ignore"):
                pin(proxy)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin_name)
    assert failed, "no pin caught mutant %s" % name
