"""CPU oracle for C = A * B^T -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, no fast-math, no
FMA contraction).  This module builds it with gcc, loads it with ctypes and
marshals numpy arrays.  ``matmul.py`` computes the same products with the
double sum taken by a library matrix product, for full-size comparisons.  ``compare`` holds the acceptance rule the parity tests
apply to a GPU result: bit-exact for integer-valued inputs, otherwise
``|C_gpu - C_ref| <= ulp_bf16(C_ref) + 1e-4 * S`` with ``S = |s| sum_k |a*b|``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
E4M3 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-fno-fast-math", "-ffp-contract=off", "-fno-builtin",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, vp, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
    lib.oracle_gemm.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                f64, f64, i32]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm_sampled.argtypes = [i32, vp, vp, i64, i64, i64, i64, i64,
                                        vp, vp, i64, f64, f64, vp, vp, i32]
    lib.oracle_gemm_sampled.restype = i32
    lib.oracle_bf16_round_n.argtypes = [vp, vp, i64]
    lib.oracle_bf16_round_n.restype = None
    lib.oracle_e4m3_table.argtypes = [vp]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_decode.restype = f64
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = f64
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_decode.restype = f64
    lib.oracle_gemm_mx.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                   i64, i32]
    lib.oracle_gemm_mx.restype = i32
    lib.oracle_gemm_mx_sampled.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                           vp, vp, i64, vp, vp, i32]
    lib.oracle_gemm_mx_sampled.restype = i32
    lib.oracle_attn_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, f64, i32,
                                    vp, i64, vp, vp, vp, vp, i32]
    lib.oracle_attn_fwd.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads to use: the affinity set, capped at 16 (one GPU's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _dtype_code(dtype) -> int:
    if dtype in (BF16, "bf16"):
        return BF16
    if dtype in (E4M3, "fp8", "e4m3"):
        return E4M3
    raise ValueError("unknown dtype %r" % (dtype,))


def _as_bits(x: np.ndarray, code: int) -> np.ndarray:
    want = np.uint16 if code == BF16 else np.uint8
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError("expected %s bit patterns, got %s" % (want, x.dtype))
    return x


def gemm(dtype, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
         lda: int | None = None, ldb: int | None = None,
         scale_a: float = 1.0, scale_b: float = 1.0, threads: int | None = None,
         want_s: bool = True):
    """Full oracle product.

    A, B are flat or 2-D arrays of bit patterns (uint16 for bf16, uint8 for
    e4m3) with row strides lda, ldb (elements).  Returns (C bits as an
    (M, N) uint16 array, S as an (M, N) float64 array or None).
    """
    code = _dtype_code(dtype)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    A = _as_bits(A, code)
    B = _as_bits(B, code)
    if M > 0 and K > 0 and A.size < (M - 1) * lda + K:
        raise ValueError("A too small")
    if N > 0 and K > 0 and B.size < (N - 1) * ldb + K:
        raise ValueError("B too small")
    C = np.zeros((M, N), dtype=np.uint16)
    S = np.zeros((M, N), dtype=np.float64) if want_s else None
    rc = _load().oracle_gemm(code, A.ctypes.data, B.ctypes.data, C.ctypes.data,
                             S.ctypes.data if S is not None else None,
                             M, N, K, lda, ldb, N, float(scale_a), float(scale_b),
                             threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return C, S


def gemm_sampled(dtype, A: np.ndarray, B: np.ndarray, M: int, N: int, K: int,
                 rows, cols, lda: int | None = None, ldb: int | None = None,
                 scale_a: float = 1.0, scale_b: float = 1.0,
                 threads: int | None = None):
    """Oracle entries C[rows[p], cols[p]] and their magnitude sums."""
    code = _dtype_code(dtype)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    A = _as_bits(A, code)
    B = _as_bits(B, code)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows/cols shape mismatch")
    n = rows.size
    c = np.zeros(n, dtype=np.uint16)
    s = np.zeros(n, dtype=np.float64)
    rc = _load().oracle_gemm_sampled(code, A.ctypes.data, B.ctypes.data, M, N, K,
                                     lda, ldb, rows.ctypes.data, cols.ctypes.data, n,
                                     float(scale_a), float(scale_b), c.ctypes.data,
                                     s.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_sampled rejected its arguments")
    return c, s


def _mx_operands(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb):
    nb = (K + 31) // 32
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldsa = nb if ldsa is None else ldsa
    ldsb = nb if ldsb is None else ldsb
    A, B = _as_bits(A, E4M3), _as_bits(B, E4M3)
    SA, SB = _as_bits(SA, E4M3), _as_bits(SB, E4M3)  # E8M0 scale bytes
    if M > 0 and K > 0 and (A.size < (M - 1) * lda + K or SA.size < (M - 1) * ldsa + nb):
        raise ValueError("A or its scales too small")
    if N > 0 and K > 0 and (B.size < (N - 1) * ldb + K or SB.size < (N - 1) * ldsb + nb):
        raise ValueError("B or its scales too small")
    return A, B, SA, SB, lda, ldb, ldsa, ldsb


def gemm_mx(A: np.ndarray, B: np.ndarray, SA: np.ndarray, SB: np.ndarray, M: int, N: int,
            K: int, lda: int | None = None, ldb: int | None = None, ldsa: int | None = None,
            ldsb: int | None = None, threads: int | None = None, want_s: bool = True):
    """Full MXFP8 oracle product.

    A, B: E4M3 bytes with row strides lda, ldb.  SA, SB: E8M0 scale bytes, one
    per 32 K-elements of a row, with row strides ldsa, ldsb (default ceil(K/32)).
    Returns (C bits (M, N) uint16, S (M, N) float64 or None).
    """
    A, B, SA, SB, lda, ldb, ldsa, ldsb = _mx_operands(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb)
    C = np.zeros((M, N), dtype=np.uint16)
    S = np.zeros((M, N), dtype=np.float64) if want_s else None
    rc = _load().oracle_gemm_mx(A.ctypes.data, B.ctypes.data, SA.ctypes.data, SB.ctypes.data,
                                C.ctypes.data, S.ctypes.data if S is not None else None,
                                M, N, K, lda, ldb, ldsa, ldsb, N, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_mx rejected its arguments")
    return C, S


def gemm_mx_sampled(A, B, SA, SB, M: int, N: int, K: int, rows, cols, lda=None, ldb=None,
                    ldsa=None, ldsb=None, threads: int | None = None):
    """MXFP8 oracle entries C[rows[p], cols[p]] and their magnitude sums."""
    A, B, SA, SB, lda, ldb, ldsa, ldsb = _mx_operands(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows/cols shape mismatch")
    n = rows.size
    c = np.zeros(n, dtype=np.uint16)
    s = np.zeros(n, dtype=np.float64)
    rc = _load().oracle_gemm_mx_sampled(A.ctypes.data, B.ctypes.data, SA.ctypes.data,
                                        SB.ctypes.data, M, N, K, lda, ldb, ldsa, ldsb,
                                        rows.ctypes.data, cols.ctypes.data, n, c.ctypes.data,
                                        s.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_mx_sampled rejected its arguments")
    return c, s


def e8m0_decode(x: int) -> float:
    """Decode one E8M0 scale byte: 2^(x - 127), NaN for 255."""
    return _load().oracle_e8m0_decode(int(x))


def bf16_round(x) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (RNE, single rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    _load().oracle_bf16_round_n(x.ctypes.data, out.ctypes.data, x.size)
    return out


def e4m3_table() -> np.ndarray:
    """The 256 decoded OCP E4M3FN values (NaN for the two NaN codes)."""
    out = np.zeros(256, dtype=np.float64)
    _load().oracle_e4m3_table(out.ctypes.data)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns to float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 values in the binade of |x|: 2^(max(floor(log2|x|), -126) - 7).

    For an exact power of two this is the spacing above it; ulp(0) = 2^-133.
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        _, e = np.frexp(ax)
    E = np.where(ax > 0, e - 1, -126)
    E = np.maximum(E, -126)
    return np.ldexp(1.0, (E - 7).astype(np.int64))


def compare(c_gpu_bits, c_ref_bits, S=None, exact: bool = False, rel_tol: float = 1e-4):
    """Apply the acceptance rule; return a dict of statistics.

    exact=True: bit equality with +0 and -0 treated as equal.
    Otherwise:  |C_gpu - C_ref| <= ulp_bf16(C_ref) + rel_tol * S, and any NaN or
    infinity in C_gpu that is not in C_ref fails.
    """
    g = np.asarray(c_gpu_bits, dtype=np.uint16).ravel()
    r = np.asarray(c_ref_bits, dtype=np.uint16).ravel()
    if g.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, r.shape))
    # equal bit patterns, or +0 against -0
    same = (g == r) | (((g & 0x7FFF) == 0) & ((r & 0x7FFF) == 0))
    stats = {"n": int(g.size), "bit_identical_frac": float(same.mean()) if g.size else 1.0,
             "neg_zero_gpu": int(np.sum(g == 0x8000))}
    if exact:
        bad = ~same
        stats.update(violations=int(bad.sum()), ok=not bool(bad.any()))
        if bad.any():
            idx = int(np.flatnonzero(bad)[0])
            stats["first_bad"] = (idx, int(g[idx]), int(r[idx]))
        return stats
    if S is None:
        raise ValueError("tolerance comparison needs S")
    S = np.asarray(S, dtype=np.float64).ravel()
    # Identical entries pass and count as 0 ulps (-1 when the identical value is
    # a NaN or an infinity); the rule is evaluated on the others only.
    d = np.flatnonzero(~same)
    gv = bf16_to_f64(g[d])
    rv = bf16_to_f64(r[d])
    Sd = S[d]
    with np.errstate(invalid="ignore"):
        err = np.abs(gv - rv)
    bound = ulp_bf16(rv) + rel_tol * Sd
    bad_d = ~(np.isfinite(gv) & (err <= bound))
    with np.errstate(divide="ignore", invalid="ignore"):
        err_f = np.where(np.isfinite(err), err, np.inf)
        ratio = np.where(bound > 0, err_f / bound, np.inf)
        rel_s = np.where(Sd > 0, err_f / Sd, np.inf)
        ulps = np.where(np.isfinite(err), np.round(err / ulp_bf16(rv)), -1)
    same_nonfinite = int(np.sum(same & ((g & 0x7F80) == 0x7F80)))
    hist = {}
    if int(same.sum()) - same_nonfinite:
        hist[0] = int(same.sum()) - same_nonfinite
    if same_nonfinite:
        hist[-1] = same_nonfinite
    u, cnt = np.unique(np.clip(ulps, -1, 8).astype(np.int64), return_counts=True)
    for a, b in zip(u.tolist(), cnt.tolist()):
        hist[int(a)] = hist.get(int(a), 0) + int(b)
    stats.update(violations=int(bad_d.sum()), ok=not bool(bad_d.any()),
                 max_err_over_bound=float(ratio.max()) if d.size else 0.0,
                 max_err_over_S=float(rel_s.max()) if d.size else 0.0,
                 ulp_hist=dict(sorted(hist.items())))
    if bad_d.any():
        k = int(np.flatnonzero(bad_d)[0])
        idx = int(d[k])
        stats["first_bad"] = (idx, int(g[idx]), int(r[idx]), float(S[idx]))
    return stats


def _strides(s, H, N, D):
    """(batch, head, token) strides in elements; None = packed B x H x N x D."""
    if s is None:
        s = (H * N * D, N * D, D)
    return np.ascontiguousarray(s, dtype=np.int64)


def attention(Q, K, V, B: int, Hq: int, Hkv: int, N: int, D: int, scale: float,
              causal: bool, q_strides=None, k_strides=None, v_strides=None, rows=None,
              threads: int | None = None):
    """Attention forward on bf16 bit patterns (uint16 arrays).

    Q is B x Hq x N x D, K and V are B x Hkv x N x D, with (batch, head, token)
    strides in elements (None = packed).  rows: flattened query rows
    (b * Hq + h) * N + i to compute, or None for all of them in order.
    Returns (O bits (nrows, D) uint16, O as float64, LSE (nrows,), A (nrows, D))
    where A = sum_j p_j |v_j| / sum_j p_j, the magnitude the tolerance uses.
    """
    Q = _as_bits(Q, BF16)
    K = _as_bits(K, BF16)
    V = _as_bits(V, BF16)
    sq = _strides(q_strides, Hq, N, D)
    sk = _strides(k_strides, Hkv, N, D)
    sv = _strides(v_strides, Hkv, N, D)
    for X, s, H in ((Q, sq, Hq), (K, sk, Hkv), (V, sv, Hkv)):
        if B * H * N > 0 and X.size < (B - 1) * s[0] + (H - 1) * s[1] + (N - 1) * s[2] + D:
            raise ValueError("operand too small for its shape and strides")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
    else:
        n = B * Hq * N
    o = np.zeros((n, D), dtype=np.uint16)
    o64 = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    amag = np.zeros((n, D), dtype=np.float64)
    rc = _load().oracle_attn_fwd(Q.ctypes.data, K.ctypes.data, V.ctypes.data, B, Hq, Hkv, N, D,
                                 sq.ctypes.data, sk.ctypes.data, sv.ctypes.data, float(scale),
                                 int(bool(causal)), rows.ctypes.data if rows is not None else None,
                                 n, o.ctypes.data, o64.ctypes.data, lse.ctypes.data,
                                 amag.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected its arguments (%d)" % rc)
    return o, o64, lse, amag
