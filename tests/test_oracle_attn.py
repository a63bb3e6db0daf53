"""Pins of the attention-forward oracle (softmax(scale * Q K^T [+ causal mask]) V
over BF16 inputs, grouped-query heads).  CPU only.

Each pin checks the oracle against something other than itself:
* torch's float64 scaled_dot_product_attention (an independent implementation;
  the oracle calls no library routine for its arithmetic), with grouped-query
  heads expanded by repeat_interleave, and torch's logsumexp for the LSE;
* 50-digit mpmath softmax attention on tiny inputs, rounded to bf16 by exact
  rational comparison: the oracle's bf16 output must be the correctly rounded
  exact value;
* closed forms: all-zero queries give the mean of the visible value rows,
  LSE = log(n) and a tolerance magnitude A equal to the mean of the visible
  values' magnitudes (A is also checked against torch's float64 softmax
  weights applied to |V|); a single key gives that key's value row exactly; the first
  causal row sees only key 0; a key that dominates by more than the double
  exponent range gives its value row exactly; a hand-derived mean that single
  rounding and double rounding (through float) round differently;
* invariants: grouped-query heads equal explicitly repeated heads bitwise, a
  scale of 2 equals doubled queries bitwise, strided storage equals packed,
  a subset of rows equals the same rows of the full result.
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from tests.test_oracle import _fraction_to_bf16_bits


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _run(oracle_mod, q, k, v, scale, causal, **kw):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    return oracle_mod.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(), B, Hq, Hkv,
                                N, D, scale, causal, **kw)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 1, 1, 1, 8), (2, 4, 2, 7, 8), (1, 2, 1, 33, 64),
                                          (1, 3, 3, 20, 16)])
def test_matches_torch_sdpa_float64(oracle_mod, B, Hq, Hkv, N, D, causal):
    q = _bf16((B, Hq, N, D), 1 + N)
    k = _bf16((B, Hkv, N, D), 2 + N)
    v = _bf16((B, Hkv, N, D), 3 + N)
    scale = D ** -0.5
    o, o64, lse, amag = _run(oracle_mod, q, k, v, scale, causal)
    rep = Hq // Hkv
    kd = k.double().repeat_interleave(rep, dim=1)
    vd = v.double().repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), kd, vd, is_causal=causal,
                                                           scale=scale)
    assert np.abs(o64 - ref.reshape(-1, D).numpy()).max() <= 1e-13
    s = (q.double() @ kd.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, dim=-1).reshape(-1).numpy()).max() <= 1e-12
    # the tolerance magnitude A = sum_j p_j |v_j| / sum_j p_j: torch's float64
    # softmax weights applied to |V| (an independent computation of the same
    # weighted mean of magnitudes)
    a_ref = torch.softmax(s, dim=-1) @ vd.abs()
    assert np.abs(amag - a_ref.reshape(-1, D).numpy()).max() <= 1e-13


def _mp_attention(q, k, v, scale, causal, dps=50):
    """Exact-ish (50 digits) attention on float64 copies of bf16 values."""
    mpmath.mp.dps = dps
    N, D = q.shape
    out = []
    for i in range(N):
        nk = i + 1 if causal else N
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, d]) * mpmath.mpf(k[j, d])
                                             for d in range(D)) for j in range(nk)]
        m = max(s)
        p = [mpmath.exp(x - m) for x in s]
        l = mpmath.fsum(p)
        out.append([mpmath.fsum(p[j] * mpmath.mpf(v[j, d]) for j in range(nk)) / l
                    for d in range(D)])
    return out


def _mpf_fraction(x):
    sign, man, exp, _ = mpmath.mpf(x)._mpf_
    return (-1 if sign else 1) * Fraction(int(man)) * (Fraction(2) ** int(exp))


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("causal", [False, True])
def test_correctly_rounded_against_mpmath(oracle_mod, seed, causal):
    N, D = 6, 4
    q = _bf16((1, 1, N, D), 100 + seed)
    k = _bf16((1, 1, N, D), 200 + seed)
    v = _bf16((1, 1, N, D), 300 + seed)
    scale = 0.5
    o, _, _, _ = _run(oracle_mod, q, k, v, scale, causal)
    exact = _mp_attention(q[0, 0].double().numpy(), k[0, 0].double().numpy(),
                          v[0, 0].double().numpy(), scale, causal)
    checked = 0
    for i in range(N):
        for d in range(D):
            x = _mpf_fraction(exact[i][d])
            want = _fraction_to_bf16_bits(x)
            # skip values within 2^-40 (relative) of a rounding boundary
            lo = _fraction_to_bf16_bits(x * (1 - Fraction(1, 2 ** 40)))
            hi = _fraction_to_bf16_bits(x * (1 + Fraction(1, 2 ** 40)))
            if lo != hi:
                continue
            assert int(o[i, d]) == want, (i, d)
            checked += 1
    assert checked >= N * D - 1


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_the_mean_of_visible_values(oracle_mod, causal):
    B, H, N, D = 1, 2, 9, 8
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    k = _bf16((B, H, N, D), 7)
    v = _bf16((B, H, N, D), 8)
    o, _, lse, amag = _run(oracle_mod, q, k, v, 0.3, causal)
    vv = v.double().numpy()
    for h in range(H):
        for i in range(N):
            n = i + 1 if causal else N
            r = h * N + i
            assert abs(lse[r] - math.log(n)) <= 1e-15 * max(1.0, math.log(n))
            for d in range(D):
                mean = sum(Fraction(float(vv[0, h, j, d])) for j in range(n)) / n
                assert int(o[r, d]) == _fraction_to_bf16_bits(mean), (h, i, d)
                # equal weights: A is the mean magnitude of the visible values
                amean = sum(abs(Fraction(float(vv[0, h, j, d]))) for j in range(n)) / n
                assert abs(Fraction(float(amag[r, d])) - amean) <= amean * Fraction(1, 2 ** 50)


def test_mean_that_double_rounding_gets_wrong(oracle_mod):
    """Hand-derived: four keys with equal scores and values 2, 2 + 2^-6, 2^-28,
    0 average to 1 + 2^-8 + 2^-30, just above a bf16 tie: rounded once it is
    1 + 2^-7 (0x3F81); through float first it would tie to 1.0 (0x3F80)."""
    vals = [2.0, 2.0 + 2.0 ** -6, 2.0 ** -28, 0.0]
    v = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).reshape(1, 1, 4, 1)
    assert [float(x) for x in v.float().ravel()] == vals
    q = torch.zeros(1, 1, 4, 1, dtype=torch.bfloat16)
    o, o64, _, _ = _run(oracle_mod, q, q.clone(), v, 1.0, False)
    assert o64[0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(o[0, 0]) == 0x3F81


def test_single_key_returns_its_value_row(oracle_mod):
    q = _bf16((2, 3, 1, 16), 11)
    k = _bf16((2, 3, 1, 16), 12)
    v = _bf16((2, 3, 1, 16), 13)
    o, _, lse, _ = _run(oracle_mod, q, k, v, 0.25, False)
    assert np.array_equal(o, _bits(v).reshape(-1, 16))
    s = 0.25 * (q.double() * k.double()).sum(-1).reshape(-1).numpy()
    assert np.abs(lse - s).max() <= 1e-15 * np.abs(s).max()


def test_first_causal_row_sees_only_key_zero(oracle_mod):
    B, H, N, D = 1, 2, 12, 8
    q, k, v = _bf16((B, H, N, D), 21), _bf16((B, H, N, D), 22), _bf16((B, H, N, D), 23)
    o, _, _, _ = _run(oracle_mod, q, k, v, 1.0, True)
    for h in range(H):
        assert np.array_equal(o[h * N], _bits(v[0, h, 0]))


def test_dominant_key_gives_its_value_row(oracle_mod):
    """Key 5 scores 2000 more than any other key: exp(-2000) underflows in
    double, so the output is key 5's value row exactly, with no overflow."""
    N, D = 8, 4
    q = torch.zeros(1, 1, N, D, dtype=torch.bfloat16)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, D, dtype=torch.bfloat16)
    k[0, 0, :, 0] = torch.tensor([-8.0, 3.0, 0.0, 1.0, -2.0, 2048.0, 4.0, 5.0])
    v = _bf16((1, 1, N, D), 31)
    o, _, lse, _ = _run(oracle_mod, q, k, v, 1.0, False)
    assert np.array_equal(o, np.tile(_bits(v[0, 0, 5]), (N, 1)))
    assert np.allclose(lse, 2048.0, rtol=0, atol=1e-12)
    # the scores themselves would overflow exp() without the max shift
    k[0, 0, 5, 0] = 65280.0  # largest bf16 below 2^16
    o, _, lse, _ = _run(oracle_mod, q, k, v, 1.0, False)
    assert np.isfinite(lse).all() and np.array_equal(o, np.tile(_bits(v[0, 0, 5]), (N, 1)))


def test_grouped_query_heads_equal_repeated_heads(oracle_mod):
    B, Hq, Hkv, N, D = 2, 6, 2, 10, 8
    q = _bf16((B, Hq, N, D), 41)
    k = _bf16((B, Hkv, N, D), 42)
    v = _bf16((B, Hkv, N, D), 43)
    for causal in (False, True):
        o, _, lse, _ = _run(oracle_mod, q, k, v, 0.35, causal)
        o2, _, lse2, _ = _run(oracle_mod, q, k.repeat_interleave(3, dim=1),
                              v.repeat_interleave(3, dim=1), 0.35, causal)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_scale_two_equals_doubled_queries(oracle_mod):
    q, k, v = _bf16((1, 2, 16, 8), 51), _bf16((1, 2, 16, 8), 52), _bf16((1, 2, 16, 8), 53)
    o, _, _, _ = _run(oracle_mod, q, k, v, 2.0, True)
    o2, _, _, _ = _run(oracle_mod, (q.float() * 2).to(torch.bfloat16), k, v, 1.0, True)
    assert np.array_equal(o, o2)


def test_strided_equals_packed(oracle_mod):
    """B x N x H x D storage with padding (NaN) between heads and tokens."""
    B, Hq, Hkv, N, D = 2, 4, 2, 6, 8
    q, k, v = _bf16((B, Hq, N, D), 61), _bf16((B, Hkv, N, D), 62), _bf16((B, Hkv, N, D), 63)
    o, _, lse, _ = _run(oracle_mod, q, k, v, 0.4, False)

    def bnhd(x, pad_h, pad_t):
        Bx, H, Nx, Dx = x.shape
        sh = Dx + pad_h
        st = H * sh + pad_t
        buf = np.full(Bx * Nx * st, 0x7FC0, dtype=np.uint16)
        xb = _bits(x)
        for b in range(Bx):
            for h in range(H):
                for t in range(Nx):
                    off = b * Nx * st + t * st + h * sh
                    buf[off:off + Dx] = xb[b, h, t]
        return buf, (Nx * st, sh, st)

    qb, sq = bnhd(q, 8, 16)
    kb, sk = bnhd(k, 0, 8)
    vb, sv = bnhd(v, 24, 0)
    o2, _, lse2, _ = oracle_mod.attention(qb, kb, vb, B, Hq, Hkv, N, D, 0.4, False,
                                          q_strides=sq, k_strides=sk, v_strides=sv)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_rows_subset_equals_full(oracle_mod):
    B, H, N, D = 2, 2, 9, 8
    q, k, v = _bf16((B, H, N, D), 71), _bf16((B, H, N, D), 72), _bf16((B, H, N, D), 73)
    o, o64, lse, a = _run(oracle_mod, q, k, v, 0.5, True)
    rows = np.array([0, 5, 17, 35, 8, 8])
    o2, o64b, lse2, a2 = _run(oracle_mod, q, k, v, 0.5, True, rows=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(lse2, lse[rows])
    assert np.array_equal(a2, a[rows]) and np.array_equal(o64b, o64[rows])
    assert (a >= np.abs(o64) - 1e-15).all()


def test_rejects_bad_arguments(oracle_mod):
    z = np.zeros(64, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.attention(z, z, z, 1, 3, 2, 2, 8, 1.0, False)  # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        oracle_mod.attention(z, z, z, 1, 1, 1, 2, 8, 1.0, False, rows=[2])
