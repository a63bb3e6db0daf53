"""GPU parity of the K-strided operand layouts (A stored K x M, B stored K x N)
through the C ABI, against the CPU oracle.

The oracle computes sum_k A(i, k) B(j, k) from the logical M x K and N x K
matrices; the GPU gets the same values stored transposed (torch transposes
them on the host, with padding columns poisoned by NaN where the stride is
wider than the matrix).  Same acceptance rule as the other parity tests:
bit-exact for integer-valued inputs, otherwise |C_gpu - C_ref| <=
ulp_bf16(C_ref) + 1e-4 * S.

Shapes cover one tile, several tiles with ragged M and N, a K tail that is
not a multiple of a stage (and, with both operands K-strided, not a multiple
of 8), more tiles than compute units (the persistent walk), the same for FP8
on its 4-wave kernel, the plain fallback (a K-strided M or N that is not
whole 16-byte chunks, for BF16 and FP8), the
A @ B convenience over torch views, and the 8192^3 workload with B stored
K x N in the benchmark's launch configuration (sampled entries).
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle
from oracle import matmul as oracle_matmul

pytestmark = pytest.mark.gpu

RTOL = 1e-4
NAN_BF16 = 0x7FC0


def _say(*a):
    print("[gpu-layouts]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _store(X, trans, ld, fill):
    """X (rows x K) as stored: rows x ld (K-contiguous) or K x ld (K-strided),
    the columns past the matrix set to the bit pattern `fill`."""
    Y = X.t() if trans else X
    r, c = Y.shape
    esz = Y.element_size()
    if esz == 2:
        out = torch.full((r, ld), fill, dtype=torch.int16).view(Y.dtype)
    else:
        out = torch.full((r, ld), fill, dtype=torch.uint8).view(Y.dtype)
    out[:, :c] = Y
    return out


def _check(dtype, A, B, M, N, K, la, lb, exact, lda=None, ldb=None, sa=1.0, sb=1.0,
           expect_kernel=None, **opts):
    """A (M x K) and B (N x K) are the logical matrices, CPU tensors."""
    lda = lda or (M if la else K)
    ldb = ldb or (N if lb else K)
    fill = NAN_BF16 if dtype == "bf16" else 0x7F
    As = _store(A, la, lda, fill).cuda()
    Bs = _store(B, lb, ldb, fill).cuda()
    dt = hk.HK_DTYPE_BF16 if dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
    C = torch.zeros((max(M, 1), N), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    plan = hk.hk_gemm_plan(dt, As, Bs, C, M, N, K, lda, ldb, N, layout_a=la, layout_b=lb, **opts)
    _say(dtype, (M, N, K), "layouts", (la, lb), "ld", (lda, ldb), plan["kernel_name"])
    if expect_kernel:
        assert plan["kernel_name"] == expect_kernel
    hk.hk_gemm_ex(dt, As, Bs, C, M, N, K, lda, ldb, N, sa, sb, layout_a=la, layout_b=lb, **opts)
    torch.cuda.synchronize()
    got = _bits16(C)[:M, :N]
    ref, S = oracle.gemm(dtype, gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)
    st = oracle.compare(got, ref, S, exact=exact, rel_tol=RTOL)
    _say("  ", "exact" if exact else "tol", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    return plan


LAYOUTS = [(0, 1), (1, 0), (1, 1)]
FAST = {(0, 1): "hk_gemm_il4_bf16_bkn", (1, 0): "hk_gemm_il4_bf16_akm",
        (1, 1): "hk_gemm_il4_bf16_akm_bkn"}


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (520, 600, 648), (8, 8, 8), (264, 1000, 1288),
                                   (1040, 776, 136), (16, 528, 4160)])
@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("integer", [True, False])
def test_bf16_layouts_full(M, N, K, layouts, integer):
    dist = "int4" if integer else "uniform"
    A = gemm_inputs.bf16_matrix(M, K, dist, 11 * M + K)
    B = gemm_inputs.bf16_matrix(N, K, dist, 13 * N + K)
    _check("bf16", A, B, M, N, K, *layouts, exact=integer, expect_kernel=FAST[layouts])


@pytest.mark.parametrize("K", [100, 1, 37, 200])
def test_bf16_both_strided_any_k(K):
    """Both operands K-strided: every K-row past K reads zero through the
    buffer bounds, so K needs no alignment on the fast path."""
    M, N = 264, 520
    A = gemm_inputs.bf16_matrix(M, K, "int4", 5 + K)
    B = gemm_inputs.bf16_matrix(N, K, "int4", 6 + K)
    _check("bf16", A, B, M, N, K, 1, 1, exact=True, expect_kernel=FAST[(1, 1)])


@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("K", [392, 1000])
def test_bf16_layouts_padded_strides_poisoned(layouts, K):
    # K = 1000: 15 whole stages, so the loop that loads interior tiles'
    # whole stages without a range check runs many times over padded rows
    M, N = 520, 264
    la, lb = layouts
    lda = (M if la else K) + 24
    ldb = (N if lb else K) + 40
    A = gemm_inputs.bf16_matrix(M, K, "normal", 71)
    B = gemm_inputs.bf16_matrix(N, K, "normal", 72)
    _check("bf16", A, B, M, N, K, la, lb, exact=False, lda=lda, ldb=ldb,
           expect_kernel=FAST[layouts])


@pytest.mark.parametrize("layouts", [(0, 1), (1, 1)])
def test_bf16_layouts_persistent_walk(layouts):
    M, N, K = 4360, 4352, 640  # 18 x 17 = 306 tiles > 256 compute units
    A = gemm_inputs.bf16_matrix(M, K, "int4", 81)
    B = gemm_inputs.bf16_matrix(N, K, "int4", 82)
    _check("bf16", A, B, M, N, K, *layouts, exact=True, expect_kernel=FAST[layouts])


@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("grid_order", ["row_major", "xcd"])
def test_bf16_layouts_grid_orders(layouts, grid_order):
    M, N, K = 1032, 1288, 256
    A = gemm_inputs.bf16_matrix(M, K, "int4", 91)
    B = gemm_inputs.bf16_matrix(N, K, "int4", 92)
    _check("bf16", A, B, M, N, K, *layouts, exact=True, grid_order=grid_order)


@pytest.mark.parametrize("layouts", LAYOUTS)
def test_bf16_layouts_basic_fallback(layouts):
    """K-strided operand rows that are not whole 16-byte chunks (601, 301)
    run on the plain kernel."""
    M, N, K = 301, 601, 136
    la, lb = layouts
    A = gemm_inputs.bf16_matrix(M, K, "uniform", 31)
    B = gemm_inputs.bf16_matrix(N, K, "uniform", 32)
    plan = _check("bf16", A, B, M, N, K, la, lb, exact=False)
    assert plan["kernel_name"] == "hk_gemm_basic_bf16"
    # and the explicit plain schedule on an aligned shape
    _check("bf16", A[:296], B[:600], 296, 600, K, la, lb, exact=False, schedule="basic",
           expect_kernel="hk_gemm_basic_bf16")


FAST8 = {(0, 1): "hk_gemm_il4_fp8_bkn", (1, 0): "hk_gemm_il4_fp8_akm",
         (1, 1): "hk_gemm_il4_fp8_akm_bkn"}


def _fp8(rows, cols, seed, integer):
    X, s = gemm_inputs.fp8_matrix(rows, cols, seed, integer)
    return X, (None if integer else s)


def _check8(M, N, K, layouts, integer, seed, **kw):
    A, sa = _fp8(M, K, seed, integer)
    B, sb = _fp8(N, K, seed + 1, integer)
    if integer:
        sa, sb = 0.5, 2.0
    return _check("fp8", A, B, M, N, K, *layouts, exact=integer, sa=sa, sb=sb, **kw)


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (528, 608, 656), (16, 16, 16),
                                   (272, 1008, 1296), (1040, 784, 144), (16, 528, 4160)])
@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("integer", [True, False])
def test_fp8_layouts_full(M, N, K, layouts, integer):
    """FP8 with K-strided operands on the 4-wave kernel (transposing 8-bit
    LDS reads): ragged tiles and K tails."""
    _check8(M, N, K, layouts, integer, 3 * M + K, expect_kernel=FAST8[layouts])


@pytest.mark.parametrize("K", [100, 1, 37, 200, 300])
def test_fp8_both_strided_any_k(K):
    """Both operands K-strided: K-rows past K read zero through the buffer
    bounds, so K needs no alignment."""
    _check8(272, 528, K, (1, 1), True, 7 + K, expect_kernel=FAST8[(1, 1)])


@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("K", [400, 1040])
def test_fp8_layouts_padded_strides_poisoned(layouts, K):
    # K = 400 is only 3 whole 128-byte stages, which never reach the loop that
    # loads interior tiles' whole stages without a range check; K = 1040 (8
    # whole stages and a tail) runs it three times over padded rows
    M, N = 528, 272
    la, lb = layouts
    lda = (M if la else K) + 32
    ldb = (N if lb else K) + 48
    _check8(M, N, K, layouts, False, 61, lda=lda, ldb=ldb, expect_kernel=FAST8[layouts])


@pytest.mark.parametrize("layouts", [(0, 1), (1, 0), (1, 1)])
def test_fp8_layouts_persistent_walk(layouts):
    _check8(4352, 4368, 640, layouts, True, 83, expect_kernel=FAST8[layouts])  # 17 x 18 tiles


@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("grid_order", ["row_major", "xcd"])
def test_fp8_layouts_grid_orders(layouts, grid_order):
    _check8(1040, 1296, 256, layouts, True, 93, grid_order=grid_order,
            expect_kernel=FAST8[layouts])


@pytest.mark.parametrize("layouts", LAYOUTS)
@pytest.mark.parametrize("integer", [True, False])
def test_fp8_layouts_basic(layouts, integer):
    """A K-strided M or N that is not a multiple of 16 runs on the plain kernel."""
    M, N, K = 264, 392, 320
    A, sa = gemm_inputs.fp8_matrix(M, K, 41, integer)
    B, sb = gemm_inputs.fp8_matrix(N, K, 42, integer)
    if integer:
        sa, sb = 0.5, 2.0
    _check("fp8", A, B, M, N, K, *layouts, exact=integer, sa=sa, sb=sb,
           expect_kernel="hk_gemm_basic_fp8")


def test_matmul_infers_layouts_from_strides():
    """hk.matmul(A, B) = A @ B for plain tensors and transposed views: each
    storage picks its layout and gives the oracle's C."""
    M, N, K = 264, 520, 200
    A = gemm_inputs.bf16_matrix(M, K, "int4", 51)   # logical A (M x K)
    Bt = gemm_inputs.bf16_matrix(N, K, "int4", 52)  # logical B^T (N x K)
    ref, _ = oracle.gemm("bf16", gemm_inputs.bits(A).ravel(), gemm_inputs.bits(Bt).ravel(), M, N, K)
    A_mk = A.cuda()
    A_km = A.t().contiguous().cuda()
    B_nk = Bt.cuda()
    B_kn = Bt.t().contiguous().cuda()
    for a_view, b_view, name in [(A_mk, B_kn, "A @ B"), (A_mk, B_nk.t(), "A @ (N x K)^T"),
                                 (A_km.t(), B_kn, "(K x M)^T @ B"),
                                 (A_km.t(), B_nk.t(), "(K x M)^T @ (N x K)^T")]:
        C = hk.matmul(a_view, b_view)
        torch.cuda.synchronize()
        st = oracle.compare(_bits16(C), ref, exact=True)
        _say("matmul", name, {k: st[k] for k in st if k != "ulp_hist"})
        assert st["ok"], (name, st)


def test_matmul_fp8_views():
    """hk.matmul on E4M3 tensors over all four storages (the 4-wave FP8
    kernels, K-strided or not), bit-exact on integer-valued inputs."""
    M, N, K = 272, 528, 208
    A, _ = gemm_inputs.fp8_matrix(M, K, 53, True)    # logical A (M x K)
    Bt, _ = gemm_inputs.fp8_matrix(N, K, 54, True)   # logical B^T (N x K)
    sa, sb = 0.5, 2.0
    ref, _ = oracle.gemm("fp8", gemm_inputs.bits(A).ravel(), gemm_inputs.bits(Bt).ravel(), M, N, K,
                         scale_a=sa, scale_b=sb)
    e4 = torch.float8_e4m3fn
    A_mk = A.view(e4).cuda()
    A_km = A.t().contiguous().view(e4).cuda()
    B_nk = Bt.view(e4).cuda()
    B_kn = Bt.t().contiguous().view(e4).cuda()
    for a_view, b_view, name in [(A_mk, B_kn, "A @ B"), (A_mk, B_nk.t(), "A @ (N x K)^T"),
                                 (A_km.t(), B_kn, "(K x M)^T @ B"),
                                 (A_km.t(), B_nk.t(), "(K x M)^T @ (N x K)^T")]:
        C = hk.matmul(a_view, b_view, scale_a=sa, scale_b=sb)
        torch.cuda.synchronize()
        st = oracle.compare(_bits16(C), ref, exact=True)
        _say("matmul fp8", name, {k: st[k] for k in st if k != "ulp_hist"})
        assert st["ok"], (name, st)


def test_bf16_8192_b_stored_kn_full_size():
    """The B-stored-K-x-N workload exactly as the benchmark launches it,
    checked on sampled entries (random plus the corners of edge tiles) with the
    oracle's loop and on every element with its matmul path."""
    w = gemm_inputs.WORKLOADS["bf16_8192_bkn"]
    x = gemm_inputs.make_inputs(w)
    A_st, B_st = gemm_inputs.stored(w, x)
    A = A_st.cuda()
    B = B_st.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    plan = hk.hk_gemm_plan(hk.HK_DTYPE_BF16, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N,
                           layout_a=w.layout_a, layout_b=w.layout_b)
    assert plan["kernel_name"] == "hk_gemm_il4_bf16_bkn"
    hk.hk_gemm_ex(hk.HK_DTYPE_BF16, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N,
                  layout_a=w.layout_a, layout_b=w.layout_b)
    torch.cuda.synchronize()
    got = _bits16(C)
    del A, B, C
    rng = np.random.default_rng(3)
    edge = np.array([0, 1, 255, 256, 4095, 4096, w.M - 256, w.M - 1])
    rows = np.concatenate([rng.integers(0, w.M, 1500), np.repeat(edge, edge.size)])
    cols = np.concatenate([rng.integers(0, w.N, 1500), np.tile(edge, edge.size)])
    ref, S = oracle.gemm_sampled("bf16", gemm_inputs.bits(x["A"]).ravel(),
                                 gemm_inputs.bits(x["B"]).ravel(), w.M, w.N, w.K, rows, cols)
    st = oracle.compare(got[rows, cols], ref, S, rel_tol=RTOL)
    _say("bf16_8192_bkn sampled", rows.size, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    ref, S = oracle_matmul.gemm_by_matmul("bf16", gemm_inputs.bits(x["A"]), gemm_inputs.bits(x["B"]),
                                          w.M, w.N, w.K)
    st = oracle.compare(got, ref, S, rel_tol=RTOL)
    _say("bf16_8192_bkn every element", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


def test_fp8_8192_b_stored_kn_full_size():
    """The FP8 B-stored-K-x-N workload as the benchmark launches it (4-wave
    kernel, transposing 8-bit reads), on sampled entries with the oracle's loop
    and on every element with its matmul path."""
    w = gemm_inputs.WORKLOADS["fp8_8192_bkn"]
    x = gemm_inputs.make_inputs(w)
    A_st, B_st = gemm_inputs.stored(w, x)
    A = A_st.cuda()
    B = B_st.cuda()
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    plan = hk.hk_gemm_plan(hk.HK_DTYPE_FP8_E4M3, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N,
                           layout_a=w.layout_a, layout_b=w.layout_b)
    assert plan["kernel_name"] == "hk_gemm_il4_fp8_bkn"
    hk.hk_gemm_ex(hk.HK_DTYPE_FP8_E4M3, A, B, C, w.M, w.N, w.K, w.lda, w.ldb, w.N,
                  x["scale_a"], x["scale_b"], layout_a=w.layout_a, layout_b=w.layout_b)
    torch.cuda.synchronize()
    got = _bits16(C)
    del A, B, C
    rng = np.random.default_rng(5)
    edge = np.array([0, 1, 255, 256, 4095, 4096, w.M - 256, w.M - 1])
    rows = np.concatenate([rng.integers(0, w.M, 1500), np.repeat(edge, edge.size)])
    cols = np.concatenate([rng.integers(0, w.N, 1500), np.tile(edge, edge.size)])
    ref, S = oracle.gemm_sampled("fp8", gemm_inputs.bits(x["A"]).ravel(),
                                 gemm_inputs.bits(x["B"]).ravel(), w.M, w.N, w.K, rows, cols,
                                 scale_a=x["scale_a"], scale_b=x["scale_b"])
    st = oracle.compare(got[rows, cols], ref, S, rel_tol=RTOL)
    _say("fp8_8192_bkn sampled", rows.size, {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    ref, S = oracle_matmul.gemm_by_matmul("fp8", gemm_inputs.bits(x["A"]), gemm_inputs.bits(x["B"]),
                                          w.M, w.N, w.K, scale_a=x["scale_a"], scale_b=x["scale_b"])
    st = oracle.compare(got, ref, S, rel_tol=RTOL)
    _say("fp8_8192_bkn every element", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
