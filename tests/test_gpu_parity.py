"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Acceptance rule (element by element): bit-exact for integer-valued inputs;
otherwise |C_gpu - C_ref| <= ulp_bf16(C_ref) + 1e-4 * S with S = |s| sum|a*b|.

* Small and medium shapes (several 256-tiles plus ragged edges and a K tail)
  are compared in full.
* Every workload at its full size runs in the launch configuration the
  benchmark times (hk_gemm_bf16 / hk_gemm_fp8 defaults) and is compared on a
  sample of entries that the oracle computes one by one (random entries plus
  the corners of every edge tile), and through properties that hold at any
  size: integer-valued inputs (bit-exact sample), identity-like B (C equals
  A exactly), a K-tail probe, and guard bands around C.
"""
import os
import sys

import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle
from oracle import matmul as oracle_matmul

pytestmark = pytest.mark.gpu

RTOL = 1e-4
SENTINEL = 0x7BAD  # a finite bf16 bit pattern no product here produces by chance


def _say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(dtype, A, B, M, N, K, lda, ldb, ldc, sa=1.0, sb=1.0, C=None, stream=None, **opts):
    """Launch through the C ABI on device tensors; returns C (bf16, rows of ldc)."""
    if C is None:
        C = torch.full((max(M, 1), ldc), 0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if opts:
        hk.hk_gemm_ex(dtype, A, B, C, M, N, K, lda, ldb, ldc, sa, sb, stream=stream, **opts)
    elif dtype == hk.HK_DTYPE_BF16:
        hk.hk_gemm_bf16(A, B, C, M, N, K, lda, ldb, ldc, stream=stream)
    else:
        hk.hk_gemm_fp8(A, B, C, M, N, K, lda, ldb, ldc, sa, sb, stream=stream)
    torch.cuda.synchronize()
    return C


def _bf16(rows, cols, dist, seed):
    return gemm_inputs.bf16_matrix(rows, cols, dist, seed)


def _full_check(dtype, A_cpu, B_cpu, M, N, K, lda, ldb, exact, sa=1.0, sb=1.0, ldc=None, **opts):
    ldc = ldc or N
    dt = hk.HK_DTYPE_BF16 if dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
    A = A_cpu.cuda()
    B = B_cpu.cuda()
    C = _run(dt, A, B, M, N, K, lda, ldb, ldc, sa, sb, **opts)
    got = _bits16(C)[:M, :N]
    ref, S = oracle.gemm(dtype, gemm_inputs.bits(A_cpu).ravel(), gemm_inputs.bits(B_cpu).ravel(),
                         M, N, K, lda=lda, ldb=ldb, scale_a=sa, scale_b=sb)
    st = oracle.compare(got, ref, S, exact=exact, rel_tol=RTOL)
    _say(dtype, (M, N, K), "exact" if exact else "tol", opts or "", {k: st[k] for k in st
                                                                  if k != "ulp_hist"})
    assert st["ok"], st
    return st


# ------------------------------------------------------------ full compares

@pytest.mark.parametrize("integer", [False, True])
def test_bf16_256_full(integer):
    w = gemm_inputs.WORKLOADS["bf16_256"]
    x = gemm_inputs.make_inputs(w, integer=integer)
    _full_check("bf16", x["A"], x["B"], 256, 256, 256, 256, 256, exact=integer)


@pytest.mark.parametrize("M,N,K", [(600, 700, 520), (257, 513, 136), (1, 1, 8), (17, 3, 64),
                                   (300, 260, 8), (64, 1000, 1288)])
@pytest.mark.parametrize("integer", [False, True])
def test_bf16_ragged_full(M, N, K, integer):
    dist = "int4" if integer else "uniform"
    A = _bf16(M, K, dist, M + K)
    B = _bf16(N, K, dist, N + K + 1)
    _full_check("bf16", A, B, M, N, K, K, K, exact=integer)


@pytest.mark.parametrize("M,N,K", [(520, 600, 640), (256, 256, 256), (300, 1, 144), (33, 513, 16)])
@pytest.mark.parametrize("integer", [False, True])
def test_fp8_ragged_full(M, N, K, integer):
    A, sa = gemm_inputs.fp8_matrix(M, K, 3 * M + K, integer)
    B, sb = gemm_inputs.fp8_matrix(N, K, 5 * N + K, integer)
    if integer:
        sa, sb = 0.5, 4.0  # powers of two keep the scaled integer sums exact
    _full_check("fp8", A, B, M, N, K, K, K, exact=integer, sa=sa, sb=sb)


# interleave8 and producer_consumer exist for BF16 only
_SCHEDULES_BY_DTYPE = [(d, s) for d in ("bf16", "fp8")
                       for s in ("pingpong8", "interleave4", "smalltile", "basic", "interleave8",
                                 "producer_consumer")
                       if d == "bf16" or s not in ("interleave8", "producer_consumer")]


@pytest.mark.parametrize("dtype,schedule", _SCHEDULES_BY_DTYPE)
@pytest.mark.parametrize("grid_order", ["row_major", "xcd"])
def test_every_variant(schedule, grid_order, dtype):
    M, N, K = 777, 1029, 512
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "normal", 11), _bf16(N, K, "normal", 12), 1.0, 1.0
    else:
        A, sa = gemm_inputs.fp8_matrix(M, K, 13)
        B, sb = gemm_inputs.fp8_matrix(N, K, 14)
    _full_check(dtype, A, B, M, N, K, K, K, exact=False, sa=sa, sb=sb, schedule=schedule,
                grid_order=grid_order)


@pytest.mark.parametrize("dtype,schedule", [(d, s) for d, s in _SCHEDULES_BY_DTYPE if s != "basic"])
@pytest.mark.parametrize("M,N,K", [(513, 769, 1040), (256, 256, 128), (300, 40, 16)])
def test_fast_schedules_ragged_integer(schedule, dtype, M, N, K):
    """Bit-exact on integer-valued inputs: edge tiles, K tails and odd stage counts."""
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "int4", M + 3), _bf16(N, K, "int4", N + 4), 1.0, 1.0
    else:
        A, _ = gemm_inputs.fp8_matrix(M, K, M + 5, integer=True)
        B, _ = gemm_inputs.fp8_matrix(N, K, N + 6, integer=True)
        sa, sb = 0.5, 4.0
    _full_check(dtype, A, B, M, N, K, K, K, exact=True, sa=sa, sb=sb, schedule=schedule)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("integer", [True, False])
def test_persistent_tile_walk_full(dtype, integer):
    """More output tiles than compute units, so that the persistent 4-wave
    kernels carry their stage pipeline from one tile into the next; ragged
    edges and a K tail (odd stage count), compared in full."""
    M, N, K = 4359, 4352, 264 if dtype == "bf16" else 656
    if dtype == "bf16":
        dist = "int4" if integer else "normal"
        A, B, sa, sb = _bf16(M, K, dist, 31), _bf16(N, K, dist, 32), 1.0, 1.0
    else:
        A, sa = gemm_inputs.fp8_matrix(M, K, 33, integer=integer)
        B, sb = gemm_inputs.fp8_matrix(N, K, 34, integer=integer)
        if integer:
            sa, sb = 0.5, 4.0
    p = hk.hk_gemm_plan(hk.HK_DTYPE_BF16 if dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3,
                        A.cuda(), B.cuda(), torch.empty(1, device="cuda"), M, N, K, K, K, N)
    assert p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4
    assert p["tiles_m"] * p["tiles_n"] > p["workgroups"]
    _full_check(dtype, A, B, M, N, K, K, K, exact=integer, sa=sa, sb=sb)


@pytest.mark.parametrize("group_m,window", [(1, 256), (3, 100), (16, 64), (8, 7)])
def test_grid_parameters(group_m, window):
    M, N, K = 1300, 1100, 256
    A = _bf16(M, K, "int4", 21)
    B = _bf16(N, K, "int4", 22)
    _full_check("bf16", A, B, M, N, K, K, K, exact=True, group_m=group_m, window=window)


def test_padded_strides_and_guard_bands():
    M, N, K, pad = 517, 300, 264, 8
    lda, ldb, ldc = K + pad, K + 2 * pad, N + pad
    A = _bf16(M, lda, "uniform", 31)
    B = _bf16(N, ldb, "uniform", 32)
    # poison the padding: a kernel that reads it gets a visibly wrong answer
    A[:, K:] = float("nan")
    B[:, K:] = float("nan")
    guard = 3
    Cbuf = torch.full(((M + 2 * guard) * ldc,), SENTINEL, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    Cv = Cbuf[guard * ldc:]
    _run(hk.HK_DTYPE_BF16, A.cuda(), B.cuda(), M, N, K, lda, ldb, ldc, C=Cv)
    allb = _bits16(Cbuf).reshape(M + 2 * guard, ldc)
    assert (allb[:guard] == SENTINEL).all() and (allb[guard + M:] == SENTINEL).all()
    body = allb[guard:guard + M]
    assert (body[:, N:] == SENTINEL).all()
    ref, S = oracle.gemm("bf16", gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(),
                         M, N, K, lda=lda, ldb=ldb)
    st = oracle.compare(body[:, :N], ref, S, rel_tol=RTOL)
    assert st["ok"], st


def test_misaligned_pointers_use_the_fallback():
    M, N, K = 130, 70, 77  # odd K: no 16-byte chunks
    A = _bf16(M, K + 1, "int4", 41)
    B = _bf16(N, K + 1, "int4", 42)
    Ad, Bd = A.cuda(), B.cuda()
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    # pointers offset by one element (2 bytes) and odd row strides
    p = hk.hk_gemm_plan(0, Ad.data_ptr() + 2, Bd.data_ptr() + 2, C, M, N, K, K + 1, K + 1, N)
    assert p["schedule"] == hk.HK_SCHEDULE_BASIC
    hk.hk_gemm_bf16(Ad.data_ptr() + 2, Bd.data_ptr() + 2, C, M, N, K, K + 1, K + 1, N)
    torch.cuda.synchronize()
    a = gemm_inputs.bits(A)[:, 1:].copy()
    b = gemm_inputs.bits(B)[:, 1:].copy()
    ref, _ = oracle.gemm("bf16", a.ravel(), b.ravel(), M, N, K)
    assert oracle.compare(_bits16(C), ref, exact=True)["ok"]


def test_odd_ldc_two_byte_stores():
    M, N, K = 70, 45, 64
    ldc = 47
    A = _bf16(M, K, "int4", 51)
    B = _bf16(N, K, "int4", 52)
    C = torch.full((M * ldc,), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    _run(hk.HK_DTYPE_BF16, A.cuda(), B.cuda(), M, N, K, K, K, ldc, C=C)
    allb = _bits16(C).reshape(M, ldc)
    assert (allb[:, N:] == SENTINEL).all()
    ref, _ = oracle.gemm("bf16", gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K)
    assert oracle.compare(allb[:, :N], ref, exact=True)["ok"]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("N", [1, 3, 4, 5, 7, 8, 9, 12, 260, 263, 264, 268, 516])
def test_sixteen_byte_stores_and_ragged_columns(dtype, N):
    """C 16-byte aligned with ldc a multiple of 8: the 4-wave kernels store
    8 columns per lane after trading halves between lane groups; a group that
    crosses N is stored column by column.  Bit-exact, padding and guard rows
    untouched."""
    M, K = 300, 192
    ldc = (N + 7) // 8 * 8 + 8
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "int4", 71), _bf16(N, K, "int4", 72), 1.0, 1.0
        dt = hk.HK_DTYPE_BF16
    else:
        A, _ = gemm_inputs.fp8_matrix(M, K, 73, integer=True)
        B, _ = gemm_inputs.fp8_matrix(N, K, 74, integer=True)
        sa, sb, dt = 0.5, 4.0, hk.HK_DTYPE_FP8_E4M3
    guard = 2
    Cbuf = torch.full(((M + 2 * guard) * ldc,), SENTINEL, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    Cv = Cbuf[guard * ldc:]
    assert Cv.data_ptr() % 16 == 0 and ldc % 8 == 0
    _say("16-byte stores", dtype, (M, N, K), "ldc", ldc)
    _run(dt, A.cuda(), B.cuda(), M, N, K, K, K, ldc, sa, sb, C=Cv, schedule="interleave4")
    allb = _bits16(Cbuf).reshape(M + 2 * guard, ldc)
    assert (allb[:guard] == SENTINEL).all() and (allb[guard + M:] == SENTINEL).all()
    body = allb[guard:guard + M]
    assert (body[:, N:] == SENTINEL).all()
    ref, _ = oracle.gemm(dtype, gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)
    st = oracle.compare(body[:, :N], ref, exact=True)
    assert st["ok"], st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("ldc_extra,c_off", [(2, 0), (4, 0), (6, 0), (8, 2), (8, 4), (8, 6), (6, 2)])
@pytest.mark.parametrize("N,schedule", [(13, "interleave4"), (264, "interleave4"),
                                        (270, "interleave4"), (270, "pingpong8")])
def test_sixteen_byte_stores_at_dword_alignment(dtype, ldc_extra, c_off, N, schedule):
    """C rows that start only 4- or 8-byte aligned (an even ldc that is not a
    multiple of 8, or C itself offset by 2, 4 or 6 elements): the 4-wave and
    ping-pong kernels still store 8 columns per lane in one 16-byte store at dword
    alignment.  Bit-exact; the columns past N, the elements before C and the
    guard rows untouched."""
    M, K = 290, 192
    ldc = (N + 7) // 8 * 8 + ldc_extra
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "int4", 75), _bf16(N, K, "int4", 76), 1.0, 1.0
        dt = hk.HK_DTYPE_BF16
    else:
        A, _ = gemm_inputs.fp8_matrix(M, K, 77, integer=True)
        B, _ = gemm_inputs.fp8_matrix(N, K, 78, integer=True)
        sa, sb, dt = 2.0, 0.25, hk.HK_DTYPE_FP8_E4M3
    guard = 2
    Cbuf = torch.full(((M + 2 * guard) * ldc + 8,), SENTINEL, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    start = guard * ldc + c_off
    Cv = Cbuf[start:]
    assert Cv.data_ptr() % 4 == 0 and ldc % 2 == 0
    assert Cv.data_ptr() % 16 != 0 or ldc % 8 != 0
    _say("dword-aligned 16-byte stores", dtype, (M, N, K), "ldc", ldc, "offset", c_off)
    _run(dt, A.cuda(), B.cuda(), M, N, K, K, K, ldc, sa, sb, C=Cv, schedule=schedule)
    allb = _bits16(Cbuf)
    assert (allb[:start] == SENTINEL).all() and (allb[start + M * ldc:] == SENTINEL).all()
    body = allb[start:start + M * ldc].reshape(M, ldc)
    assert (body[:, N:] == SENTINEL).all()
    ref, _ = oracle.gemm(dtype, gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)
    st = oracle.compare(body[:, :N], ref, exact=True)
    assert st["ok"], st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_k_order_does_not_change_exact_results(dtype):
    """The 4-wave kernels walk K in a per-chiplet rotated order (chiplet
    w mod 8 starts w mod 8 eighths of the way in).  Changing the tile order
    moves tiles to other chiplets and so changes their K order: on
    integer-valued inputs every order must give the oracle's bits.  K has a
    tail and a whole-stage count that is not a multiple of 8."""
    M, N, K = 1100, 700, 1000 if dtype == "bf16" else 1936
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "int4", 81), _bf16(N, K, "int4", 82), 1.0, 1.0
        dt = hk.HK_DTYPE_BF16
    else:
        A, _ = gemm_inputs.fp8_matrix(M, K, 83, integer=True)
        B, _ = gemm_inputs.fp8_matrix(N, K, 84, integer=True)
        sa, sb, dt = 0.5, 4.0, hk.HK_DTYPE_FP8_E4M3
    ref, _ = oracle.gemm(dtype, gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)
    Ad, Bd = A.cuda(), B.cuda()
    for opts in (dict(grid_order="xcd"), dict(grid_order="row_major"),
                 dict(grid_order="xcd", group_m=1), dict(grid_order="xcd", window=24)):
        _say("K order", dtype, (M, N, K), opts)
        C = _run(dt, Ad, Bd, M, N, K, K, K, N, sa, sb, schedule="interleave4", **opts)
        st = oracle.compare(_bits16(C), ref, exact=True)
        assert st["ok"], (opts, st)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M", [768, 769])
def test_interior_and_edge_tiles_with_padded_rows(dtype, M):
    """The 4-wave kernels load the whole K stages of a tile that lies inside
    C without a range check; edge tiles and the K tail keep the checked
    loads.  With every tile inside C (M = 768, N = 512) and with a row of
    edge tiles (M = 769), operands whose rows are padded past K with a poison
    value must give the oracle's bits on integer-valued inputs: no load may
    read the padding."""
    N = 512
    K, pad = (1000, 8) if dtype == "bf16" else (1936, 16)
    if dtype == "bf16":
        A, B, sa, sb = _bf16(M, K, "int4", 91), _bf16(N, K, "int4", 92), 1.0, 1.0
        dt = hk.HK_DTYPE_BF16
    else:
        A, _ = gemm_inputs.fp8_matrix(M, K, 93, integer=True)
        B, _ = gemm_inputs.fp8_matrix(N, K, 94, integer=True)
        sa, sb, dt = 0.5, 4.0, hk.HK_DTYPE_FP8_E4M3
    ref, _ = oracle.gemm(dtype, gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)

    def padded(X):
        P = torch.full((X.shape[0], K + pad), 64.0).to(X.dtype)
        P[:, :K] = X
        return P.cuda()

    _say("interior/edge tiles, padded rows", dtype, (M, N, K), "ld", K + pad)
    C = _run(dt, padded(A), padded(B), M, N, K, K + pad, K + pad, N, sa, sb,
             schedule="interleave4")
    st = oracle.compare(_bits16(C), ref, exact=True)
    assert st["ok"], st


def test_zero_k_writes_zeros_and_empty_is_noop():
    C = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    hk.hk_gemm_bf16(0, 0, C, 5, 7, 0, 1, 1, 7)
    torch.cuda.synchronize()
    assert (C.float() == 0).all()
    D = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    hk.hk_gemm_bf16(0, 0, D, 0, 7, 16, 16, 16, 7)
    hk.hk_gemm_fp8(0, 0, D, 5, 0, 16, 16, 16, 7, 1.0, 1.0)
    torch.cuda.synchronize()
    assert (D.float() == 3).all()


def test_non_default_stream():
    M, N, K = 512, 384, 320
    A = _bf16(M, K, "int4", 61).cuda()
    B = _bf16(N, K, "int4", 62).cuda()
    s = torch.cuda.Stream()
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        hk.hk_gemm_bf16(A, B, C, M, N, K, K, K, N, stream=s)
    s.synchronize()
    ref, _ = oracle.gemm("bf16", _bits16(A).ravel(), _bits16(B).ravel(), M, N, K)
    assert oracle.compare(_bits16(C), ref, exact=True)["ok"]


def test_repeatable_bitwise():
    M, N, K = 1024, 768, 1024
    A = _bf16(M, K, "normal", 71).cuda()
    B = _bf16(N, K, "normal", 72).cuda()
    C1 = _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N)
    C2 = _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


# -------------------------------------------------------- full-size workloads

def _edge_samples(M, N, tile, rng, n_random):
    """Random entries plus the four corners of every tile row/column edge."""
    rows = [rng.integers(0, M, n_random)]
    cols = [rng.integers(0, N, n_random)]
    tm = np.arange(0, M, tile)
    tn = np.arange(0, N, tile)
    for r in np.unique(np.concatenate([tm, np.minimum(tm + tile - 1, M - 1)])):
        for c in (0, N - 1, rng.integers(0, N)):
            rows.append([r]); cols.append([c])
    for c in np.unique(np.concatenate([tn, np.minimum(tn + tile - 1, N - 1)])):
        for r in (0, M - 1, rng.integers(0, M)):
            rows.append([r]); cols.append([c])
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def _sampled_check(w, x, integer, n_random=3000):
    M, N, K = w.M, w.N, w.K
    dt = hk.HK_DTYPE_BF16 if w.dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
    sa, sb = x["scale_a"], x["scale_b"]
    if integer and w.dtype == "fp8":
        sa, sb = 0.5, 4.0
    A, B = x["A"].cuda(), x["B"].cuda()
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _say("launch", w.name, "integer" if integer else w.dist, (M, N, K))
    if dt == hk.HK_DTYPE_BF16:
        hk.hk_gemm_bf16(A, B, C, M, N, K, K, K, N)
    else:
        hk.hk_gemm_fp8(A, B, C, M, N, K, K, K, N, sa, sb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.index * 7 + int(integer))
    rows, cols = _edge_samples(M, N, 256, rng, n_random)
    got = _bits16(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
    ref, S = oracle.gemm_sampled(w.dtype, gemm_inputs.bits(x["A"]).ravel(),
                                 gemm_inputs.bits(x["B"]).ravel(), M, N, K, rows, cols,
                                 scale_a=sa, scale_b=sb)
    st = oracle.compare(got, ref, S, exact=integer, rel_tol=RTOL)
    _say(w.name, "sampled", rows.size, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    return C


FULL = ["bf16_4096", "bf16_8192", "bf16_mlp", "bf16_mlp_ragged", "fp8_8192"]


@pytest.mark.parametrize("name", FULL)
@pytest.mark.parametrize("integer", [False, True])
def test_full_size_sampled(name, integer):
    w = gemm_inputs.WORKLOADS[name]
    x = gemm_inputs.make_inputs(w, integer=integer)
    _sampled_check(w, x, integer)


@pytest.mark.parametrize("name", ["bf16_8192", "bf16_mlp_ragged", "fp8_8192"])
def test_full_size_identity_like_B(name):
    """B[j, k] = 1 if j == k else 0 (j < min(N, K)): C[:, :min(N,K)] == A exactly."""
    w = gemm_inputs.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    sa_seed, _ = w.seeds()
    if w.dtype == "bf16":
        A = gemm_inputs.bf16_matrix(M, K, w.dist, sa_seed).cuda()
        B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
        d = min(N, K)
        B[torch.arange(d), torch.arange(d)] = 1.0
        C = _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N)
        want = A[:, :d]
    else:
        A8, sa = gemm_inputs.fp8_matrix(M, K, sa_seed)
        A = A8.cuda()
        B = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
        d = min(N, K)
        B[torch.arange(d), torch.arange(d)] = 0x38  # e4m3 1.0
        C = _run(hk.HK_DTYPE_FP8_E4M3, A, B, M, N, K, K, K, N, 2.0 ** -4, 8.0)
        # 2^-4 * 8 = 0.5: every e4m3 value times 0.5 is an exact bf16 value
        dec = oracle.e4m3_table()[gemm_inputs.bits(A8)[:, :d]] * 0.5
        want = torch.from_numpy(oracle.bf16_round(dec).view(np.int16)).cuda()
    # +0 and -0 compare equal: an e4m3 -0 times 1 summed from +0 is +0
    st = oracle.compare(_bits16(C[:, :d]), _bits16(want), exact=True)
    ok = st["ok"]
    rest_zero = bool((C[:, d:].float() == 0).all()) if N > d else True
    _say(name, "identity-like B", ok, rest_zero)
    assert ok and rest_zero


def test_k_tail_probe_ragged():
    """Only the last 8 K positions of B are non-zero, so C is exactly the tail sum."""
    w = gemm_inputs.WORKLOADS["bf16_mlp_ragged"]
    M, N, K = w.M, w.N, w.K
    A_cpu = gemm_inputs.bf16_matrix(M, K, "int4", 81)
    B_cpu = torch.zeros((N, K), dtype=torch.bfloat16)
    B_cpu[:, K - 8:] = gemm_inputs.bf16_matrix(N, 8, "int4", 82)
    C = _run(hk.HK_DTYPE_BF16, A_cpu.cuda(), B_cpu.cuda(), M, N, K, K, K, N)
    rng = np.random.default_rng(5)
    rows, cols = _edge_samples(M, N, 256, rng, 4000)
    got = _bits16(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
    ref, _ = oracle.gemm_sampled("bf16", gemm_inputs.bits(A_cpu).ravel(),
                                 gemm_inputs.bits(B_cpu).ravel(), M, N, K, rows, cols)
    st = oracle.compare(got, ref, exact=True)
    assert st["ok"], st
    assert np.count_nonzero(ref) > 0.5 * ref.size  # the probe really exercises the tail


# ---------------------------------------------------------------- clock record
#
# hk_gemm_opts.clock_stamps: the persistent kernels write, for workgroups 0-7, the
# shader-clock and constant-rate counters at their start and end.  The record
# must leave the product untouched and write nothing outside its 32 words.

STAMP_SENTINEL = 0x5A5A5A5A5A5A5A5A


@pytest.mark.parametrize("schedule", ["interleave4", "pingpong8"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_clock_record_leaves_results_unchanged(dtype, schedule):
    M, N, K = 1024, 2048, 512  # 32 tiles: every chiplet gets a first workgroup
    if dtype == "bf16":
        A_cpu, B_cpu = _bf16(M, K, "int4", 71), _bf16(N, K, "int4", 72)
        dt, sa, sb = hk.HK_DTYPE_BF16, 1.0, 1.0
    else:
        A_cpu = gemm_inputs.fp8_matrix(M, K, 73, integer=True)[0]
        B_cpu = gemm_inputs.fp8_matrix(N, K, 74, integer=True)[0]
        dt, sa, sb = hk.HK_DTYPE_FP8_E4M3, 0.5, 4.0
    A, B = A_cpu.cuda(), B_cpu.cuda()
    stamps = torch.full((40,), STAMP_SENTINEL, dtype=torch.int64, device="cuda")
    plain = _run(dt, A, B, M, N, K, K, K, N, sa, sb, schedule=schedule)
    rec = _run(dt, A, B, M, N, K, K, K, N, sa, sb, schedule=schedule, clock_stamps=stamps)
    assert torch.equal(_as_i16(plain), _as_i16(rec))
    st = stamps.cpu().tolist()
    assert st[32:] == [STAMP_SENTINEL] * 8
    ghz = hk.chiplet_clocks_ghz(st[:32], hk.hk_wall_clock_khz())
    _say("clock record", dtype, schedule, [None if g is None else round(g, 3) for g in ghz])
    for x in range(8):
        t0, r0, t1, r1 = st[4 * x:4 * x + 4]
        assert STAMP_SENTINEL not in (t0, r0, t1, r1) and t1 > t0 and r1 > r0, (x, st)
        assert 0.3 < ghz[x] < 3.5, ghz


def _as_i16(C):
    return C.view(torch.int16)


def test_clock_record_untouched_without_those_workgroups_or_schedule():
    # two tiles: only workgroups 0 and 1 exist; BASIC never writes the record
    M, N, K = 256, 512, 256
    A, B = _bf16(M, K, "int4", 75).cuda(), _bf16(N, K, "int4", 76).cuda()
    stamps = torch.full((32,), STAMP_SENTINEL, dtype=torch.int64, device="cuda")
    _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N, schedule="interleave4", clock_stamps=stamps)
    st = stamps.cpu().tolist()
    assert STAMP_SENTINEL not in st[:8]
    assert st[8:] == [STAMP_SENTINEL] * 24
    stamps.fill_(STAMP_SENTINEL)
    _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N, schedule="basic", clock_stamps=stamps)
    assert stamps.cpu().tolist() == [STAMP_SENTINEL] * 32


# ------------------------------------------------------- full-size, compared in full
#
# 4096^3 costs the oracle about 15 s on 16 host threads, so it is compared
# element by element, random and integer-valued, in the launch configuration
# the benchmark times.  At 8192^3 whole 256-row tile bands (the first, an
# interior one chosen by seed, and the last) are compared against the oracle.
# Integer-valued inputs have one exact product whatever the summation order
# (every partial sum is an integer far below 2^53), so at 8192^3 and on the
# MLP shape every output element is also checked bit for bit against a
# float64 product of the same integers, rounded once to bf16 (on the ragged
# shape too, where every edge tile and the K tail of 8 take part).

def _launch_default(w, x, sa=None, sb=None, **opts):
    M, N, K = w.M, w.N, w.K
    A, B = x["A"].cuda(), x["B"].cuda()
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sa = x["scale_a"] if sa is None else sa
    sb = x["scale_b"] if sb is None else sb
    _say("launch", w.name, (M, N, K), opts or "bench launch configuration")
    if opts:
        dt = hk.HK_DTYPE_BF16 if w.dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
        hk.hk_gemm_ex(dt, A, B, C, M, N, K, K, K, N, sa, sb, **opts)
    elif w.dtype == "bf16":
        hk.hk_gemm_bf16(A, B, C, M, N, K, K, K, N)
    else:
        hk.hk_gemm_fp8(A, B, C, M, N, K, K, K, N, sa, sb)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("integer", [False, True])
def test_bf16_4096_compared_in_full(integer):
    w = gemm_inputs.WORKLOADS["bf16_4096"]
    x = gemm_inputs.make_inputs(w, integer=integer)
    C = _launch_default(w, x)
    got = _bits16(C)
    ref, S = oracle.gemm("bf16", gemm_inputs.bits(x["A"]).ravel(), gemm_inputs.bits(x["B"]).ravel(),
                         w.M, w.N, w.K)
    st = oracle.compare(got, ref, S, exact=integer, rel_tol=RTOL)
    _say("bf16_4096 full", "integer" if integer else w.dist,
         {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


def _tile_bands(M, rng):
    interior = int(rng.integers(1, M // 256 - 1)) * 256
    return [0, interior, M - 256]


@pytest.mark.parametrize("schedule", [None, "pingpong8"])
def test_bf16_8192_tile_bands_against_the_oracle(schedule):
    w = gemm_inputs.WORKLOADS["bf16_8192"]
    x = gemm_inputs.make_inputs(w)
    C = _launch_default(w, x, **({"schedule": schedule} if schedule else {}))
    Ab, Bb = gemm_inputs.bits(x["A"]), gemm_inputs.bits(x["B"])
    for r0 in _tile_bands(w.M, np.random.default_rng(11)):
        ref, S = oracle.gemm("bf16", np.ascontiguousarray(Ab[r0:r0 + 256]).ravel(), Bb.ravel(),
                             256, w.N, w.K)
        st = oracle.compare(_bits16(C[r0:r0 + 256]), ref, S, rel_tol=RTOL)
        _say("bf16_8192", schedule or "default", "rows", r0, r0 + 255,
             {k: st[k] for k in st if k != "ulp_hist"})
        assert st["ok"], (r0, st)


def _exact_integer_product(A_cpu, B_cpu, scale=1.0):
    """bf16 bits of scale * A B^T for integer-valued operands, computed exactly."""
    a = A_cpu.to(torch.float64) if A_cpu.dtype == torch.bfloat16 else \
        torch.from_numpy(oracle.e4m3_table()[gemm_inputs.bits(A_cpu)])
    b = B_cpu.to(torch.float64) if B_cpu.dtype == torch.bfloat16 else \
        torch.from_numpy(oracle.e4m3_table()[gemm_inputs.bits(B_cpu)])
    prod = (a @ b.t()) * scale
    assert float(prod.abs().max()) < 2.0 ** 24  # every sum is exact in fp32 too
    return oracle.bf16_round(prod.numpy())


@pytest.mark.parametrize("name,schedule", [("bf16_8192", None), ("bf16_8192", "pingpong8"),
                                           ("bf16_mlp", None), ("bf16_mlp_ragged", None),
                                           ("fp8_8192", None)])
def test_full_size_integer_exact_everywhere(name, schedule):
    w = gemm_inputs.WORKLOADS[name]
    x = gemm_inputs.make_inputs(w, integer=True)
    sa, sb = (0.5, 4.0) if w.dtype == "fp8" else (1.0, 1.0)
    C = _launch_default(w, x, sa, sb, **({"schedule": schedule} if schedule else {}))
    want = _exact_integer_product(x["A"], x["B"], sa * sb)
    got = _bits16(C)
    same = (got == want) | (((got | want) & 0x7FFF) == 0)  # +0 and -0 are equal
    bad = int((~same).sum())
    _say(name, schedule or "default", "integer-valued, every element exact:", bad == 0, bad)
    assert bad == 0


@pytest.mark.parametrize("name,schedule", [("bf16_8192", None), ("bf16_8192", "pingpong8"),
                                           ("bf16_mlp", None), ("fp8_8192", None)])
def test_full_size_random_compared_in_full(name, schedule):
    """Random inputs at full size, every output element against the oracle
    (its matmul path, pinned to the loop on the CPU)."""
    w = gemm_inputs.WORKLOADS[name]
    x = gemm_inputs.make_inputs(w)
    C = _launch_default(w, x, **({"schedule": schedule} if schedule else {}))
    got = _bits16(C)
    del C
    ref, S = oracle_matmul.gemm_by_matmul(w.dtype, gemm_inputs.bits(x["A"]), gemm_inputs.bits(x["B"]),
                                          w.M, w.N, w.K, scale_a=x["scale_a"], scale_b=x["scale_b"])
    st = oracle.compare(got, ref, S, rel_tol=RTOL)
    _say(name, schedule or "default", "every element", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


def test_pingpong8_8192_sampled():
    w = gemm_inputs.WORKLOADS["bf16_8192"]
    x = gemm_inputs.make_inputs(w)
    C = _launch_default(w, x, schedule="pingpong8")
    rng = np.random.default_rng(13)
    rows, cols = _edge_samples(w.M, w.N, 256, rng, 3000)
    got = _bits16(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
    ref, S = oracle.gemm_sampled("bf16", gemm_inputs.bits(x["A"]).ravel(),
                                 gemm_inputs.bits(x["B"]).ravel(), w.M, w.N, w.K, rows, cols)
    st = oracle.compare(got, ref, S, rel_tol=RTOL)
    _say("bf16_8192 pingpong8 sampled", rows.size, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


# ------------------------------------------------------------------ repacking
#
# Operands whose rows straddle cache lines can be copied to a padded stride
# in a caller-provided workspace first.  The copy changes neither the tile
# walk nor the K order, so the result must be bit-identical to the call on
# the operands as given, and it must match the oracle.

def _ws_tensor(nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K,pad", [(600, 700, 520, 8), (257, 513, 136, 24), (1030, 300, 1040, 40)])
@pytest.mark.parametrize("schedule", ["auto", "pingpong8"])
def test_repack_always_matches_oracle_and_direct(dtype, M, N, K, pad, schedule):
    if dtype == "fp8":
        # the fast schedules take FP8 rows in whole 16-byte chunks
        K, pad = 16 * ((K + 15) // 16), 16 * ((pad + 15) // 16)
        A_cpu, sa = gemm_inputs.fp8_matrix(M, K + pad, 91)
        B_cpu, sb = gemm_inputs.fp8_matrix(N, K + pad, 92)
        dt = hk.HK_DTYPE_FP8_E4M3
    else:
        A_cpu, B_cpu = _bf16(M, K + pad, "uniform", 91), _bf16(N, K + pad, "uniform", 92)
        sa = sb = 1.0
        dt = hk.HK_DTYPE_BF16
    lda = ldb = K + pad  # rows of lda bytes (times the element size) straddle lines
    A, B = A_cpu.cuda(), B_cpu.cuda()
    need = hk.hk_gemm_workspace_size(dt, A, B, A, M, N, K, lda, ldb, N, schedule=schedule,
                                     repack="always")
    assert need > 0
    ws = _ws_tensor(need)
    direct = _run(dt, A, B, M, N, K, lda, ldb, N, sa, sb, schedule=schedule, repack="never")
    rep = _run(dt, A, B, M, N, K, lda, ldb, N, sa, sb, schedule=schedule, repack="always",
               workspace=ws)
    assert torch.equal(direct.view(torch.int16), rep.view(torch.int16))
    ref, S = oracle.gemm(dtype, gemm_inputs.bits(A_cpu).ravel(), gemm_inputs.bits(B_cpu).ravel(),
                         M, N, K, lda=lda, ldb=ldb, scale_a=sa, scale_b=sb)
    st = oracle.compare(_bits16(rep)[:M, :N], ref, S, rel_tol=RTOL)
    _say("repack", dtype, schedule, (M, N, K, lda), need, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("which", ["A", "B"])
def test_repack_one_operand(dtype, which):
    """Only one operand's rows straddle cache lines: the copy launch takes that
    operand's rows alone, and the workspace holds that copy alone."""
    M, N, K = 520, 610, 272
    esz = 2 if dtype == "bf16" else 1
    aligned = 320 if dtype == "bf16" else 384   # rows of whole 128-byte lines
    straddle = K + 16                           # 576 or 288 bytes: not whole lines
    assert (aligned * esz) % 128 == 0 and (straddle * esz) % 128 != 0
    lda, ldb = (straddle, aligned) if which == "A" else (aligned, straddle)
    if dtype == "fp8":
        A_cpu, sa = gemm_inputs.fp8_matrix(M, lda, 93)
        B_cpu, sb = gemm_inputs.fp8_matrix(N, ldb, 94)
        dt = hk.HK_DTYPE_FP8_E4M3
    else:
        A_cpu, B_cpu = _bf16(M, lda, "uniform", 93), _bf16(N, ldb, "uniform", 94)
        sa = sb = 1.0
        dt = hk.HK_DTYPE_BF16
    A, B = A_cpu.cuda(), B_cpu.cuda()
    need = hk.hk_gemm_workspace_size(dt, A, B, A, M, N, K, lda, ldb, N, repack="always")
    rows = M if which == "A" else N
    padded = (K * esz + 1023) // 1024 * 1024
    padded += 1024 if padded % 8192 == 0 else 0
    assert need == (rows * padded + 255) // 256 * 256, (need, rows, padded)
    ws = _ws_tensor(need)
    direct = _run(dt, A, B, M, N, K, lda, ldb, N, sa, sb, repack="never")
    rep = _run(dt, A, B, M, N, K, lda, ldb, N, sa, sb, repack="always", workspace=ws)
    assert torch.equal(direct.view(torch.int16), rep.view(torch.int16))
    ref, S = oracle.gemm(dtype, gemm_inputs.bits(A_cpu).ravel(), gemm_inputs.bits(B_cpu).ravel(),
                         M, N, K, lda=lda, ldb=ldb, scale_a=sa, scale_b=sb)
    st = oracle.compare(_bits16(rep)[:M, :N], ref, S, rel_tol=RTOL)
    _say("repack one operand", dtype, which, need, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


def test_ragged_full_size_with_workspace():
    """The ragged MLP shape in the launch configuration the bench times for it:
    hk_gemm_ex with a workspace, which copies both operands (16 400-byte rows)
    to 17 KiB rows.  Bit-identical to the direct call, compared with the
    oracle on every element (and on a sample with its loop), and
    integer-valued inputs exact everywhere."""
    w = gemm_inputs.WORKLOADS["bf16_mlp_ragged"]
    M, N, K = w.M, w.N, w.K
    fake = 1 << 20  # the query only looks at alignment
    need = hk.hk_gemm_workspace_size(hk.HK_DTYPE_BF16, fake, fake, fake, M, N, K, K, K, N)
    assert need > 0
    ws = _ws_tensor(need)
    for integer in (False, True):
        x = gemm_inputs.make_inputs(w, integer=integer)
        A, B = x["A"].cuda(), x["B"].cuda()
        _say("launch", w.name, "with workspace", need, "integer" if integer else w.dist)
        rep = _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N, workspace=ws)
        direct = _run(hk.HK_DTYPE_BF16, A, B, M, N, K, K, K, N, repack="never")
        assert torch.equal(direct.view(torch.int16), rep.view(torch.int16))
        del direct
        if integer:
            want = _exact_integer_product(x["A"], x["B"])
            got = _bits16(rep)
            bad = int((~((got == want) | (((got | want) & 0x7FFF) == 0))).sum())
            _say(w.name, "repacked, integer-valued, every element exact:", bad == 0, bad)
            assert bad == 0
        else:
            rng = np.random.default_rng(17)
            rows, cols = _edge_samples(M, N, 256, rng, 3000)
            got = _bits16(rep[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
            ref, S = oracle.gemm_sampled("bf16", gemm_inputs.bits(x["A"]).ravel(),
                                         gemm_inputs.bits(x["B"]).ravel(), M, N, K, rows, cols)
            st = oracle.compare(got, ref, S, rel_tol=RTOL)
            _say(w.name, "repacked, sampled", rows.size, {k: st[k] for k in st if k != "ulp_hist"})
            assert st["ok"], st
            got = _bits16(rep)
            ref, S = oracle_matmul.gemm_by_matmul("bf16", gemm_inputs.bits(x["A"]),
                                                  gemm_inputs.bits(x["B"]), M, N, K)
            st = oracle.compare(got, ref, S, rel_tol=RTOL)
            _say(w.name, "repacked, every element", {k: st[k] for k in st if k != "ulp_hist"})
            assert st["ok"], st
