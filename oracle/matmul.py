"""The oracle products with the double-precision sum taken by a library matrix product.
TEST INFRASTRUCTURE ONLY, like the rest of this package.

Same definition as ``oracle.c`` (the textbook product C = A * B^T that the pages
"HipKittens: fast and furious AMD kernels", section "Performance results", and
"How to make AMD GPUs go brrr", section "Real kernel example", name without
writing it out):

    C[i][j] = RNE_bf16( s * sum_k dec(A[i][k]) * dec(B[j][k]) )
    S[i][j] = |s| * sum_k |dec(A[i][k]) * dec(B[j][k])|

with s = 1 for BF16, s = sA * sB for FP8 with per-tensor scales, and for MXFP8
each element multiplied by its block's E8M0 scale before the product (OCP MX
v1.0, blocks of 32 along K).  Decoding is exact (bf16 widened to double, e4m3
and e8m0 from the loop oracle's pinned tables), every element product is exact
in double, the scale is applied once and the result is rounded once, by the
loop oracle's pinned RNE routine.

The one difference from the loop oracle is the order of the double additions:
numpy's matrix product (a BLAS dgemm) blocks the sum over k.  The two results
differ by a few double roundings, about K * 2^-53 of S, so they round to the
same bf16 value unless the exact sum lies that close to a bf16 rounding
boundary.  This is what makes a full-size comparison cost seconds instead of
minutes.  The loop oracle stays the reference; these functions are pinned to
it and to the same closed forms and fixtures in the CPU tests.

``attention_by_matmul`` does the same for the attention forward (the pages'
second workload: "How to make AMD GPUs go brrr", section "Real kernel example";
"HipKittens", section "Performance results"): textbook scaled dot-product
attention over BF16 inputs, its scores and weighted sums over a block of query
rows taken by library matrix products.
"""
from __future__ import annotations

import numpy as np

import oracle


def _rows(X: np.ndarray, rows: int, K: int, ld: int) -> np.ndarray:
    """View a flat array of bit patterns as rows x K with row stride ld (elements)."""
    X = np.ascontiguousarray(X).ravel()
    if rows == 0 or K == 0:
        return np.zeros((rows, K), dtype=X.dtype)
    return np.lib.stride_tricks.as_strided(X, shape=(rows, K), strides=(ld * X.itemsize, X.itemsize),
                                           writeable=False)


def _decode(code: int, X: np.ndarray, r0: int, r1: int, K: int, ld: int, tab) -> np.ndarray:
    """Rows [r0, r1) of an operand, decoded exactly to double."""
    flat = np.ascontiguousarray(X).ravel()
    v = _rows(flat[r0 * ld:], r1 - r0, K, ld)
    if code == oracle.BF16:
        return oracle.bf16_to_f64(v)
    return tab[v]


def gemm_by_matmul(dtype, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                   lda: int | None = None, ldb: int | None = None,
                   scale_a: float = 1.0, scale_b: float = 1.0, want_s: bool = True,
                   rows_per_chunk: int = 1024):
    """The product of ``oracle.gemm`` (same arguments and results) with a library dgemm."""
    code = oracle._dtype_code(dtype)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    A = oracle._as_bits(A, code)
    B = oracle._as_bits(B, code)
    if K > 0 and ((M > 0 and (lda < K or A.size < (M - 1) * lda + K)) or
                  (N > 0 and (ldb < K or B.size < (N - 1) * ldb + K))):
        raise ValueError("operand too small for its shape and stride")
    tab = oracle.e4m3_table() if code == oracle.E4M3 else None
    s = float(scale_a) * float(scale_b) if code == oracle.E4M3 else 1.0
    b = _decode(code, B, 0, N, K, ldb, tab)
    b_abs = np.abs(b) if want_s else None
    C = np.zeros((M, N), dtype=np.uint16)
    S = np.zeros((M, N), dtype=np.float64) if want_s else None
    for r0 in range(0, M, rows_per_chunk):
        r1 = min(r0 + rows_per_chunk, M)
        a = _decode(code, A, r0, r1, K, lda, tab)
        # + 0.0: the loop sums from +0.0, so a zero sum is +0 there whatever the
        # library's order gives
        C[r0:r1] = oracle.bf16_round(((a @ b.T) + 0.0) * s)
        if want_s:
            S[r0:r1] = (np.abs(a) @ b_abs.T) * abs(s)
    return C, S


def _decode_mx(X, SX, r0, r1, K, ld, lds, tab, xtab) -> np.ndarray:
    """Rows [r0, r1) of an MXFP8 operand: element value times its block's scale, in double."""
    nb = (K + 31) // 32
    v = tab[_rows(np.ascontiguousarray(X).ravel()[r0 * ld:], r1 - r0, K, ld)]
    x = xtab[_rows(np.ascontiguousarray(SX).ravel()[r0 * lds:], r1 - r0, nb, lds)]
    return v * np.repeat(x, 32, axis=1)[:, :K]


def gemm_mx_by_matmul(A: np.ndarray, B: np.ndarray, SA: np.ndarray, SB: np.ndarray, M: int,
                      N: int, K: int, lda: int | None = None, ldb: int | None = None,
                      ldsa: int | None = None, ldsb: int | None = None, want_s: bool = True,
                      rows_per_chunk: int = 1024):
    """The product of ``oracle.gemm_mx`` (same arguments and results) with a library dgemm."""
    A, B, SA, SB, lda, ldb, ldsa, ldsb = oracle._mx_operands(A, B, SA, SB, M, N, K, lda, ldb,
                                                            ldsa, ldsb)
    tab = oracle.e4m3_table()
    xtab = np.array([oracle.e8m0_decode(x) for x in range(256)], dtype=np.float64)
    b = _decode_mx(B, SB, 0, N, K, ldb, ldsb, tab, xtab)
    b_abs = np.abs(b) if want_s else None
    C = np.zeros((M, N), dtype=np.uint16)
    S = np.zeros((M, N), dtype=np.float64) if want_s else None
    for r0 in range(0, M, rows_per_chunk):
        r1 = min(r0 + rows_per_chunk, M)
        a = _decode_mx(A, SA, r0, r1, K, lda, ldsa, tab, xtab)
        C[r0:r1] = oracle.bf16_round((a @ b.T) + 0.0)
        if want_s:
            S[r0:r1] = np.abs(a) @ b_abs.T
    return C, S


def _head(X: np.ndarray, s, b: int, h: int, N: int, D: int) -> np.ndarray:
    """The N x D token rows of head (b, h), decoded exactly to double."""
    flat = np.ascontiguousarray(X).ravel()
    if N == 0:
        return np.zeros((0, D), dtype=np.float64)
    off = int(b * s[0] + h * s[1])
    v = np.lib.stride_tricks.as_strided(flat[off:], shape=(N, D),
                                        strides=(int(s[2]) * flat.itemsize, flat.itemsize),
                                        writeable=False)
    return oracle.bf16_to_f64(v)


def attention_by_matmul(Q, K, V, B: int, Hq: int, Hkv: int, N: int, D: int, scale: float,
                        causal: bool, q_strides=None, k_strides=None, v_strides=None, rows=None,
                        rows_per_chunk: int = 512):
    """The attention forward of ``oracle.attention`` (same arguments and results).

    The loop oracle's steps on a block of query rows at a time: scores
    s_j = scale * q . k_j by a library matrix product (keys past the query
    masked out when causal), m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j,
    O = RNE_bf16(sum_j p_j v_j / l), LSE = m + log(l) and the tolerance
    magnitude A = sum_j p_j |v_j| / l.  Query head h reads key/value head
    h / (Hq / Hkv).  Only the order of the double additions differs.
    """
    Q = oracle._as_bits(Q, oracle.BF16)
    K = oracle._as_bits(K, oracle.BF16)
    V = oracle._as_bits(V, oracle.BF16)
    if B < 0 or Hq < 1 or Hkv < 1 or N < 0 or D < 1 or Hq % Hkv != 0:
        raise ValueError("invalid attention shape")
    sq = oracle._strides(q_strides, Hq, N, D)
    sk = oracle._strides(k_strides, Hkv, N, D)
    sv = oracle._strides(v_strides, Hkv, N, D)
    for X, s, H in ((Q, sq, Hq), (K, sk, Hkv), (V, sv, Hkv)):
        if B * H * N > 0 and X.size < (B - 1) * s[0] + (H - 1) * s[1] + (N - 1) * s[2] + D:
            raise ValueError("operand too small for its shape and strides")
    total = B * Hq * N
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= total):
            raise ValueError("row index out of range")
    o = np.zeros((total, D), dtype=np.uint16)
    o64 = np.zeros((total, D), dtype=np.float64)
    lse = np.zeros(total, dtype=np.float64)
    amag = np.zeros((total, D), dtype=np.float64)
    group = Hq // Hkv
    keys = np.arange(N)
    for b in range(B):
        for kvh in range(Hkv):
            k = _head(K, sk, b, kvh, N, D)
            v = _head(V, sv, b, kvh, N, D)
            v_abs = np.abs(v)
            for h in range(kvh * group, (kvh + 1) * group):
                q = _head(Q, sq, b, h, N, D)
                base = (b * Hq + h) * N
                for i0 in range(0, N, rows_per_chunk):
                    i1 = min(i0 + rows_per_chunk, N)
                    # with the causal mask no row of the block sees a key past i1 - 1
                    nk = i1 if causal else N
                    s = (q[i0:i1] @ k[:nk].T) * scale
                    if causal:
                        s[keys[None, :nk] > np.arange(i0, i1)[:, None]] = -np.inf
                    m = s.max(axis=1)
                    p = np.exp(s - m[:, None])
                    l = p.sum(axis=1)
                    val = (p @ v[:nk]) / l[:, None]
                    o64[base + i0:base + i1] = val
                    o[base + i0:base + i1] = oracle.bf16_round(val)
                    amag[base + i0:base + i1] = (p @ v_abs[:nk]) / l[:, None]
                    lse[base + i0:base + i1] = m + np.log(l)
    if rows is not None:
        return o[rows], o64[rows], lse[rows], amag[rows]
    return o, o64, lse, amag
