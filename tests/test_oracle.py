"""Pins for the CPU oracle: each test ties it to something other than itself.

* hand-derived fixtures (tests/golden/oracle_cases.txt);
* the OCP E4M3FN table against torch's float8_e4m3fn decoder and the closed
  form's landmark codes;
* the double -> bf16 rounding against torch's float -> bf16 cast on
  float-representable inputs, plus cases that only single rounding gets right;
* integer-valued products against an int64 matrix product (exact);
* exact rational sums (fractions.Fraction) on tiny shapes;
* identity B, transpose identity, padded strides, and the magnitude sum S.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "oracle_cases.txt")


def _parse_golden():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        rest = rest.strip()
        if key == "case":
            cur = {"name": rest}
            cases.append(cur)
        elif key == "dtype":
            f = rest.split()
            cur.update(dtype=f[0], M=int(f[1]), N=int(f[2]), K=int(f[3]),
                       sa=float(f[4]), sb=float(f[5]))
        elif key in ("A", "B", "C"):
            cur[key] = [int(x, 16) for x in rest.split()]
        elif key == "why":
            cur["why"] = rest
    return cases


GOLDEN_CASES = _parse_golden()


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=[c["name"] for c in GOLDEN_CASES])
def test_golden_fixture(oracle_mod, case):
    bt = np.uint16 if case["dtype"] == "bf16" else np.uint8
    A = np.array(case["A"], dtype=bt)
    B = np.array(case["B"], dtype=bt)
    C, _ = oracle_mod.gemm(case["dtype"], A, B, case["M"], case["N"], case["K"],
                           scale_a=case["sa"], scale_b=case["sb"], threads=1)
    assert C.ravel().tolist() == case["C"], case["why"]


def test_golden_file_has_cases():
    assert len(GOLDEN_CASES) >= 12


# ---------------------------------------------------------------- e4m3 decode

def test_e4m3_table_matches_torch(oracle_mod):
    tab = oracle_mod.e4m3_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float32).double().numpy()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    assert np.array_equal(np.signbit(tab[ok]), np.signbit(ref[ok]))


def test_e4m3_landmarks(oracle_mod):
    tab = oracle_mod.e4m3_table()
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x07] == 7 * 2.0 ** -9
    assert tab[0x08] == 2.0 ** -6          # smallest normal
    assert tab[0x38] == 1.0 and tab[0x40] == 2.0
    assert tab[0x80] == 0.0 and math.copysign(1.0, tab[0x80]) == -1.0
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert int(np.isnan(tab).sum()) == 2
    finite = tab[~np.isnan(tab)]
    assert finite.max() == 448.0


# --------------------------------------------------------------- bf16 rounding

def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(f32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_random_patterns(oracle_mod):
    rng = np.random.default_rng(12345)
    u = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    got = oracle_mod.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, _torch_bf16_bits(f))


def test_bf16_round_matches_torch_ties_and_edges(oracle_mod):
    hi = np.arange(0, 2 ** 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    got = oracle_mod.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, _torch_bf16_bits(f))


def test_bf16_round_single_rounding_cases(oracle_mod):
    x = np.array([
        1.0 + 2.0 ** -8 + 2.0 ** -40,      # just above a tie: up
        1.0 + 2.0 ** -8 - 2.0 ** -40,      # just below a tie: down
        -(1.0 + 2.0 ** -8 + 2.0 ** -40),
        (2.0 - 2.0 ** -8) * 2.0 ** 127,    # tie at the top: overflows to inf
        (2.0 - 2.0 ** -8 - 2.0 ** -30) * 2.0 ** 127,  # below it: largest finite
        2.0 ** -134 + 2.0 ** -170,         # above half the smallest subnormal
        float("nan"), float("inf"), -0.0,
    ])
    got = oracle_mod.bf16_round(x).tolist()
    assert got == [0x3F81, 0x3F80, 0xBF81, 0x7F80, 0x7F7F, 0x0001, 0x7FC0, 0x7F80, 0x8000]


# ------------------------------------------------------- integer-valued, exact

def _int_operands(rng, rows, cols, ld, lo=-4, hi=4):
    v = rng.integers(lo, hi + 1, size=(rows, cols))
    full = np.zeros((rows, ld), dtype=np.int64)
    full[:, :cols] = v
    full[:, cols:] = 7  # padding that must never be read
    return v, full


def _exact_int_to_bf16(v: np.ndarray) -> np.ndarray:
    # |v| < 2^24, so int64 -> float32 is exact and torch's float32 -> bf16 cast
    # (round to nearest even) gives the single correct rounding.
    assert np.abs(v).max(initial=0) < 2 ** 24
    return _torch_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("M,N,K,pad", [(1, 1, 1, 0), (3, 5, 7, 0), (17, 9, 33, 3),
                                       (64, 48, 200, 8), (5, 70, 1024, 0)])
def test_integer_bf16_exact(oracle_mod, M, N, K, pad):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a, afull = _int_operands(rng, M, K, K + pad)
    b, bfull = _int_operands(rng, N, K, K + pad)
    A = _torch_bf16_bits(afull.astype(np.float32))
    B = _torch_bf16_bits(bfull.astype(np.float32))
    C, S = oracle_mod.gemm("bf16", A, B, M, N, K, lda=K + pad, ldb=K + pad)
    ref = a @ b.T
    assert np.array_equal(C, _exact_int_to_bf16(ref))
    assert np.array_equal(S, (np.abs(a) @ np.abs(b).T).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(4, 4, 16), (33, 17, 300), (8, 64, 1000)])
def test_integer_fp8_exact_with_power_of_two_scales(oracle_mod, M, N, K):
    rng = np.random.default_rng(K)
    a = rng.integers(-16, 17, size=(M, K))
    b = rng.integers(-16, 17, size=(N, K))
    # integers up to 16 in magnitude are exact e4m3 values
    A = torch.from_numpy(a.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    B = torch.from_numpy(b.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sa, sb = 0.25, 8.0
    C, S = oracle_mod.gemm("fp8", A, B, M, N, K, scale_a=sa, scale_b=sb)
    ref = (a @ b.T) * 2  # sa * sb = 2
    assert np.array_equal(C, _exact_int_to_bf16(ref))
    assert np.array_equal(S, (np.abs(a) @ np.abs(b).T).astype(np.float64) * 2)


def test_integer_from_the_workload_generator(oracle_mod):
    w = gemm_inputs.WORKLOADS["bf16_256"]
    x = gemm_inputs.make_inputs(w, integer=True)
    A, B = x["A"], x["B"]
    M, N, K = 96, 80, w.K
    a = A[:M].float().numpy().astype(np.int64)
    b = B[:N].float().numpy().astype(np.int64)
    C, _ = oracle_mod.gemm("bf16", gemm_inputs.bits(A[:M]), gemm_inputs.bits(B[:N]), M, N, K)
    assert np.array_equal(C, _exact_int_to_bf16(a @ b.T))


# ------------------------------------------------ exact rationals, tiny shapes

def _fraction_to_bf16_bits(x: Fraction) -> int:
    """Round an exact rational to bf16 (RNE) by exact comparison."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    ax = abs(x)
    E = math.floor(math.log2(ax))           # fix up float error below
    while Fraction(2) ** E > ax:
        E -= 1
    while Fraction(2) ** (E + 1) <= ax:
        E += 1
    E = max(E, -126)
    q = Fraction(2) ** (E - 7)
    n = ax / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(val))
    assert Fraction(float(f)) == val
    return sign | (int(f.view(np.uint32)) >> 16)


def _bf16_fraction(bits: int) -> Fraction:
    return Fraction(float((np.uint32(bits) << 16).view(np.float32)))


def _random_bf16_bits(rng, n, lo_exp=-12, hi_exp=4):
    sign = rng.integers(0, 2, n) << 15
    exp = rng.integers(127 + lo_exp, 127 + hi_exp, n) << 7
    frac = rng.integers(0, 128, n)
    return (sign | exp | frac).astype(np.uint16)


@pytest.mark.parametrize("seed", range(6))
def test_fraction_bruteforce_bf16(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    for M, N, K in [(1, 1, 1), (2, 3, 5), (4, 4, 16), (3, 2, 9)]:
        A = _random_bf16_bits(rng, M * K)
        B = _random_bf16_bits(rng, N * K)
        C, S = oracle_mod.gemm("bf16", A, B, M, N, K)
        for i in range(M):
            for j in range(N):
                tot = sum((_bf16_fraction(A[i * K + k]) * _bf16_fraction(B[j * K + k])
                           for k in range(K)), Fraction(0))
                assert int(C[i, j]) == _fraction_to_bf16_bits(tot), (M, N, K, i, j)
                mag = sum((abs(_bf16_fraction(A[i * K + k]) * _bf16_fraction(B[j * K + k]))
                           for k in range(K)), Fraction(0))
                assert S[i, j] == float(mag)


def test_fraction_bruteforce_ties(oracle_mod):
    """Sums constructed to land exactly on bf16 midpoints in several binades."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        e = int(rng.integers(-20, 20))
        m = int(rng.integers(128, 256))         # 8-bit significand
        base = m * 2.0 ** (e - 7)
        half = 2.0 ** (e - 8)                   # half a quantum at this binade
        vals = np.array([base, half], dtype=np.float32)
        A = _torch_bf16_bits(vals)
        B = np.array([0x3F80, 0x3F80], dtype=np.uint16)
        C, _ = oracle_mod.gemm("bf16", A, B, 1, 1, 2)
        want = _fraction_to_bf16_bits(Fraction(base) + Fraction(half))
        assert int(C[0, 0]) == want
        assert (want & 1) == 0   # a tie always lands on an even significand


@pytest.mark.parametrize("seed", range(4))
def test_fraction_bruteforce_fp8(oracle_mod, seed):
    rng = np.random.default_rng(200 + seed)
    tab = oracle_mod.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    for M, N, K in [(1, 1, 3), (2, 2, 8), (3, 4, 16)]:
        A = rng.choice(codes, M * K)
        B = rng.choice(codes, N * K)
        sa = float(np.float32(rng.uniform(0.01, 3)))
        sb = float(np.float32(rng.uniform(0.01, 3)))
        C, _ = oracle_mod.gemm("fp8", A, B, M, N, K, scale_a=sa, scale_b=sb)
        for i in range(M):
            for j in range(N):
                tot = sum((Fraction(tab[A[i * K + k]]) * Fraction(tab[B[j * K + k]])
                           for k in range(K)), Fraction(0))
                tot = tot * Fraction(sa) * Fraction(sb)
                # exact value of the definition, rounded once; the oracle's one
                # inexact step (acc * (sa*sb) in double) cannot move it here
                assert int(C[i, j]) == _fraction_to_bf16_bits(tot), (M, N, K, i, j)


# ------------------------------------------------------ layout and identities

def test_identity_B_bf16(oracle_mod):
    rng = np.random.default_rng(3)
    M, K = 37, 29
    A = _random_bf16_bits(rng, M * K, -30, 30)
    I = np.zeros((K, K), dtype=np.uint16)
    I[np.arange(K), np.arange(K)] = 0x3F80
    C, _ = oracle_mod.gemm("bf16", A, I, M, K, K)
    assert np.array_equal(C, A.reshape(M, K))


def test_identity_B_fp8_power_of_two_scales(oracle_mod):
    rng = np.random.default_rng(4)
    M, K = 23, 19
    tab = oracle_mod.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    A = rng.choice(codes, M * K)
    one = 0x38
    I = np.zeros((K, K), dtype=np.uint8)
    I[np.arange(K), np.arange(K)] = one
    sa, sb = 2.0 ** -3, 2.0 ** 5
    C, _ = oracle_mod.gemm("fp8", A, I, M, K, K, scale_a=sa, scale_b=sb)
    ref = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float32) * (sa * sb)
    ref = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(M, K)
    C = np.where(C == 0x8000, 0, C)
    ref = np.where(ref == 0x8000, 0, ref)
    assert np.array_equal(C, ref)


def test_transpose_identity_all_tiny_shapes(oracle_mod):
    rng = np.random.default_rng(5)
    tab = oracle_mod.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    for M, N, K in itertools.product(range(1, 7), repeat=3):
        A = _random_bf16_bits(rng, M * K)
        B = _random_bf16_bits(rng, N * K)
        C1, S1 = oracle_mod.gemm("bf16", A, B, M, N, K, threads=1)
        C2, S2 = oracle_mod.gemm("bf16", B, A, N, M, K, threads=1)
        assert np.array_equal(C1, C2.T) and np.array_equal(S1, S2.T)
        A8 = rng.choice(codes, M * K)
        B8 = rng.choice(codes, N * K)
        D1, _ = oracle_mod.gemm("fp8", A8, B8, M, N, K, scale_a=0.5, scale_b=3.0, threads=1)
        D2, _ = oracle_mod.gemm("fp8", B8, A8, N, M, K, scale_a=3.0, scale_b=0.5, threads=1)
        assert np.array_equal(D1, D2.T)


def test_non_square_orientation(oracle_mod):
    """A is M x K and B is N x K: a transposed-operand mistake changes this."""
    M, N, K = 2, 3, 4
    a = np.arange(1, M * K + 1).reshape(M, K)
    b = np.arange(-N * K // 2, N * K - N * K // 2).reshape(N, K)
    A = _torch_bf16_bits(a.astype(np.float32).ravel())
    B = _torch_bf16_bits(b.astype(np.float32).ravel())
    C, _ = oracle_mod.gemm("bf16", A, B, M, N, K)
    assert np.array_equal(C, _exact_int_to_bf16(a @ b.T))


def test_strided_equals_packed(oracle_mod):
    rng = np.random.default_rng(6)
    M, N, K, pad = 19, 23, 45, 5
    A = _random_bf16_bits(rng, M * (K + pad)).reshape(M, K + pad)
    B = _random_bf16_bits(rng, N * (K + pad)).reshape(N, K + pad)
    C1, S1 = oracle_mod.gemm("bf16", A.ravel(), B.ravel(), M, N, K, lda=K + pad, ldb=K + pad)
    C2, S2 = oracle_mod.gemm("bf16", np.ascontiguousarray(A[:, :K]).ravel(),
                             np.ascontiguousarray(B[:, :K]).ravel(), M, N, K)
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def test_sampled_equals_full(oracle_mod):
    rng = np.random.default_rng(8)
    M, N, K = 40, 50, 70
    A = _random_bf16_bits(rng, M * K)
    B = _random_bf16_bits(rng, N * K)
    C, S = oracle_mod.gemm("bf16", A, B, M, N, K)
    rows = rng.integers(0, M, 100)
    cols = rng.integers(0, N, 100)
    c, s = oracle_mod.gemm_sampled("bf16", A, B, M, N, K, rows, cols)
    assert np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])


def test_zero_k_gives_plus_zero(oracle_mod):
    A = np.zeros(0, dtype=np.uint16)
    C, S = oracle_mod.gemm("bf16", A, A, 3, 4, 0)
    assert not C.any() and not S.any()


def test_rejects_bad_arguments(oracle_mod):
    A = np.zeros(16, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.gemm("bf16", A, A, 2, 2, 4, lda=3)
    with pytest.raises(ValueError):
        oracle_mod.gemm_sampled("bf16", A, A, 2, 2, 4, [2], [0])


# ------------------------------------------------------------- the comparator

def test_compare_rule(oracle_mod):
    ref = np.array([0x3F80, 0x3F80, 0x3F80, 0x0000], dtype=np.uint16)
    S = np.array([1.0, 1.0, 1000.0, 0.0])
    # one ulp off at 1.0 passes; two ulps fail unless S is large
    gpu = np.array([0x3F81, 0x3F82, 0x3F82, 0x8000], dtype=np.uint16)
    st = oracle_mod.compare(gpu, ref, S)
    assert st["violations"] == 1 and st["first_bad"][0] == 1
    st = oracle_mod.compare(ref, ref, exact=True)
    assert st["ok"]
    st = oracle_mod.compare(np.array([0x8000], np.uint16), np.array([0], np.uint16), exact=True)
    assert st["ok"]
    nan = oracle_mod.compare(np.array([0x7FC0], np.uint16), np.array([0x3F80], np.uint16),
                             np.array([1e6]))
    assert not nan["ok"]


def _rule_one(g: int, r: int, s: float, rel_tol: float):
    """The acceptance rule for one element, written out: (ok, ulps or -1, err/bound)."""
    gv = float(oracle_bits_to_f64(g))
    rv = float(oracle_bits_to_f64(r))
    if g == r or (g & 0x7FFF) == 0 == (r & 0x7FFF):
        return True, (0 if math.isfinite(gv) else -1), 0.0
    err = abs(gv - rv)
    ax = abs(rv)
    E = max(math.frexp(ax)[1] - 1, -126) if ax > 0 and math.isfinite(ax) else -126
    ulp = 2.0 ** (E - 7)
    bound = ulp + rel_tol * s
    ok = math.isfinite(gv) and err <= bound
    ulps = round(err / ulp) if math.isfinite(err) else -1
    ratio = err / bound if math.isfinite(err) else math.inf
    return ok, ulps, ratio


def oracle_bits_to_f64(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def test_compare_matches_the_rule_element_by_element(oracle_mod):
    """The comparator against the rule evaluated one element at a time, on
    identical, nearby, signed-zero, NaN and infinite entries."""
    rng = np.random.default_rng(21)
    n = 3000
    r = _random_bf16_bits(rng, n, -20, 20)
    g = r.copy()
    kind = rng.integers(0, 8, n)
    step = rng.integers(1, 4, n).astype(np.uint16)
    g = np.where(kind == 1, r + step, g)
    g = np.where(kind == 2, r - step, g)
    g = np.where(kind == 3, r ^ 0x8000, g)                 # sign flipped
    g = np.where(kind == 4, np.uint16(0x7FC0), g)          # NaN on the GPU side
    r = np.where(kind == 5, np.uint16(0x7F80), r)          # infinity in the reference
    g = np.where(kind == 6, np.uint16(0x8000), g)
    r = np.where(kind == 6, np.uint16(0x0000), r)          # -0 against +0
    g = g.astype(np.uint16)
    r = r.astype(np.uint16)
    S = np.where(rng.random(n) < 0.2, 0.0, np.abs(rng.standard_normal(n)) * 2.0 ** rng.integers(-20, 20, n))
    st = oracle_mod.compare(g, r, S, rel_tol=1e-4)
    want = [_rule_one(int(a), int(b), float(c), 1e-4) for a, b, c in zip(g, r, S)]
    bad = [i for i, w in enumerate(want) if not w[0]]
    assert st["violations"] == len(bad) and st["ok"] == (not bad)
    assert st["first_bad"][0] == bad[0]
    hist = {}
    for _, u, _ in want:
        u = min(max(u, -1), 8)
        hist[u] = hist.get(u, 0) + 1
    assert st["ulp_hist"] == dict(sorted(hist.items()))
    assert st["max_err_over_bound"] == max(w[2] for w in want)
    assert st["bit_identical_frac"] == sum(1 for a, b in zip(g, r)
                                            if a == b or (a & 0x7FFF) == 0 == (b & 0x7FFF)) / n
