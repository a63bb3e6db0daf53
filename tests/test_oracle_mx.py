"""Pins of the MXFP8 oracle (OCP MX v1.0: E4M3 elements, one E8M0 scale per 32
K-elements of a row).  CPU only.

Each pin checks the oracle against something other than itself:
* unit scales reduce it to the plain FP8 product, which test_oracle.py pins;
* exact rational sums over tiny shapes, with partial last blocks, the element
  values decoded by torch's float8_e4m3fn and the scales as exact powers of two;
* integer-valued elements with small power-of-two scales, whose sums are exact
  in float64 whatever the order, against a torch float64 matmul of the
  dequantised operands rounded by torch's float -> bf16 cast;
* single nonzero terms on both sides of every block boundary (block index k / 32);
* a NaN scale poisons exactly the rows or columns that use it;
* strided storage of elements and scales, sampled entries, argument checks.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.test_oracle import _fraction_to_bf16_bits


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN bytes with torch (independent of the oracle's table)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _nb(K):
    return (K + 31) // 32


def test_unit_scales_equal_plain_fp8(oracle_mod):
    rng = np.random.default_rng(1)
    codes = _finite_codes()
    for M, N, K in [(5, 7, 64), (3, 4, 100), (8, 2, 33)]:
        A = rng.choice(codes, M * K)
        B = rng.choice(codes, N * K)
        SA = np.full(M * _nb(K), 127, dtype=np.uint8)
        SB = np.full(N * _nb(K), 127, dtype=np.uint8)
        C, S = oracle_mod.gemm_mx(A, B, SA, SB, M, N, K)
        C0, S0 = oracle_mod.gemm("fp8", A, B, M, N, K, scale_a=1.0, scale_b=1.0)
        assert np.array_equal(C, C0)
        assert np.array_equal(S, S0)


@pytest.mark.parametrize("seed", range(4))
def test_fraction_bruteforce(oracle_mod, seed):
    rng = np.random.default_rng(300 + seed)
    codes = _finite_codes()
    for M, N, K in [(1, 1, 1), (2, 3, 31), (2, 2, 32), (3, 2, 33), (2, 2, 96), (1, 3, 100)]:
        nb = _nb(K)
        A = rng.choice(codes, M * K)
        B = rng.choice(codes, N * K)
        SA = rng.integers(112, 143, M * nb).astype(np.uint8)
        SB = rng.integers(112, 143, N * nb).astype(np.uint8)
        av, bv = _torch_e4m3(A), _torch_e4m3(B)
        C, S = oracle_mod.gemm_mx(A, B, SA, SB, M, N, K)
        for i in range(M):
            for j in range(N):
                tot = Fraction(0)
                mag = Fraction(0)
                for k in range(K):
                    xa = Fraction(2) ** (int(SA[i * nb + k // 32]) - 127)
                    xb = Fraction(2) ** (int(SB[j * nb + k // 32]) - 127)
                    p = xa * Fraction(av[i * K + k]) * xb * Fraction(bv[j * K + k])
                    tot += p
                    mag += abs(p)
                assert int(C[i, j]) == _fraction_to_bf16_bits(tot), (M, N, K, i, j)
                # S is a double sum with one rounding per add: within K ulps
                assert abs(Fraction(S[i, j]) - mag) <= mag * K * Fraction(2) ** -52


def test_integer_valued_against_torch_matmul(oracle_mod):
    """Elements in {-4..4}, scales 2^-4..2^4: every partial sum is a multiple of
    2^-8 below 2^17, exact in float64 in any order and in float32, so torch's
    float64 matmul followed by its float32 -> bf16 cast rounds exactly once."""
    rng = np.random.default_rng(11)
    vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], dtype=np.float32)
    for M, N, K in [(33, 17, 96), (20, 40, 160), (7, 9, 32)]:
        nb = _nb(K)
        a = rng.choice(vals, (M, K))
        b = rng.choice(vals, (N, K))
        A = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().ravel()
        B = torch.from_numpy(b).to(torch.float8_e4m3fn).view(torch.uint8).numpy().ravel()
        SA = rng.integers(123, 132, (M, nb)).astype(np.uint8)
        SB = rng.integers(123, 132, (N, nb)).astype(np.uint8)
        xa = np.repeat(np.ldexp(1.0, SA.astype(np.int64) - 127), 32, axis=1)[:, :K]
        xb = np.repeat(np.ldexp(1.0, SB.astype(np.int64) - 127), 32, axis=1)[:, :K]
        ref = torch.from_numpy(a.astype(np.float64) * xa) @ torch.from_numpy(
            (b.astype(np.float64) * xb).T.copy())
        want = ref.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        C, _ = oracle_mod.gemm_mx(A, B, SA.ravel(), SB.ravel(), M, N, K)
        assert np.array_equal(C, want)


def test_block_boundaries(oracle_mod):
    """One nonzero term at k: C = X_A(block of k) * X_B(block of k) * a * b."""
    K = 130  # blocks [0,32) [32,64) [64,96) [96,128) [128,130)
    nb = _nb(K)
    one = 0x38  # E4M3 1.0
    SA = np.array([120, 121, 122, 123, 124], dtype=np.uint8)
    SB = np.array([130, 132, 134, 136, 138], dtype=np.uint8)
    for k in [0, 31, 32, 63, 64, 95, 96, 127, 128, 129]:
        A = np.zeros(K, dtype=np.uint8)
        B = np.zeros(K, dtype=np.uint8)
        A[k] = one
        B[k] = one
        C, _ = oracle_mod.gemm_mx(A, B, SA, SB, 1, 1, K)
        e = int(SA[k // 32]) + int(SB[k // 32]) - 254
        want = int(torch.tensor(2.0 ** e, dtype=torch.float32).to(torch.bfloat16)
                   .view(torch.int16).item()) & 0xFFFF
        assert int(C[0, 0]) == want, k
    assert nb == 5


def test_nan_scale_poisons_its_row_only(oracle_mod):
    rng = np.random.default_rng(5)
    codes = _finite_codes()
    M, N, K = 4, 3, 64
    A = rng.choice(codes, M * K)
    B = rng.choice(codes, N * K)
    SA = np.full(M * 2, 127, dtype=np.uint8)
    SB = np.full(N * 2, 127, dtype=np.uint8)
    SA[2 * 2 + 1] = 255  # row 2, second block
    C, _ = oracle_mod.gemm_mx(A, B, SA, SB, M, N, K)
    nan_rows = {i for i in range(M) for j in range(N)
                if (C[i, j] & 0x7F80) == 0x7F80 and (C[i, j] & 0x7F) != 0}
    assert nan_rows == {2}
    SB[1 * 2 + 0] = 255  # column 1, first block
    C, _ = oracle_mod.gemm_mx(A, B, SA, SB, M, N, K)
    for i in range(M):
        for j in range(N):
            is_nan = (C[i, j] & 0x7F80) == 0x7F80 and (C[i, j] & 0x7F) != 0
            assert is_nan == (i == 2 or j == 1), (i, j)


def test_e8m0_values(oracle_mod):
    assert oracle_mod.e8m0_decode(127) == 1.0
    assert oracle_mod.e8m0_decode(128) == 2.0
    assert oracle_mod.e8m0_decode(0) == 2.0 ** -127
    assert oracle_mod.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(oracle_mod.e8m0_decode(255))


def test_strided_equals_packed(oracle_mod):
    rng = np.random.default_rng(9)
    codes = _finite_codes()
    M, N, K = 6, 5, 96
    nb = _nb(K)
    A = rng.choice(codes, (M, K))
    B = rng.choice(codes, (N, K))
    SA = rng.integers(120, 135, (M, nb)).astype(np.uint8)
    SB = rng.integers(120, 135, (N, nb)).astype(np.uint8)
    C0, S0 = oracle_mod.gemm_mx(A.ravel(), B.ravel(), SA.ravel(), SB.ravel(), M, N, K)
    Ap = np.full((M, K + 16), 0x7F, dtype=np.uint8)  # NaN padding must never be read
    Bp = np.full((N, K + 48), 0x7F, dtype=np.uint8)
    SAp = np.full((M, nb + 5), 255, dtype=np.uint8)
    SBp = np.full((N, nb + 1), 255, dtype=np.uint8)
    Ap[:, :K], Bp[:, :K], SAp[:, :nb], SBp[:, :nb] = A, B, SA, SB
    C1, S1 = oracle_mod.gemm_mx(Ap.ravel(), Bp.ravel(), SAp.ravel(), SBp.ravel(), M, N, K,
                                lda=K + 16, ldb=K + 48, ldsa=nb + 5, ldsb=nb + 1)
    assert np.array_equal(C0, C1)
    assert np.array_equal(S0, S1)


def test_sampled_equals_full(oracle_mod):
    rng = np.random.default_rng(13)
    codes = _finite_codes()
    M, N, K = 9, 11, 70
    nb = _nb(K)
    A = rng.choice(codes, M * K)
    B = rng.choice(codes, N * K)
    SA = rng.integers(120, 135, M * nb).astype(np.uint8)
    SB = rng.integers(120, 135, N * nb).astype(np.uint8)
    C, S = oracle_mod.gemm_mx(A, B, SA, SB, M, N, K)
    rows = rng.integers(0, M, 40)
    cols = rng.integers(0, N, 40)
    c, s = oracle_mod.gemm_mx_sampled(A, B, SA, SB, M, N, K, rows, cols)
    assert np.array_equal(c, C[rows, cols])
    assert np.array_equal(s, S[rows, cols])


def test_rejects_short_scale_rows(oracle_mod):
    A = np.zeros(64, dtype=np.uint8)
    S = np.zeros(4, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle_mod.gemm_mx(A, A, S, S, 1, 1, 64, ldsa=1)
