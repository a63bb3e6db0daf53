"""FP8 per-tensor scales read from device memory (hk_gemm_opts.scale_a_dev,
scale_b_dev), through the C ABI.

The kernel reads the device fp32 values when it runs and forms the same fp32
product as the host does for by-value scales, so equal values must give the
same bits as a by-value call, on every FP8 schedule and layout.  One call per
schedule is also checked against the oracle with those values, and a captured
HIP graph must pick up scale values written between its replays.
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu
RTOL = 1e-4
FP8 = hk.HK_DTYPE_FP8_E4M3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _say(*a):
    print("[gpu-dev-scales]", *a, flush=True)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _dev(x):
    return torch.tensor([x], dtype=torch.float32, device="cuda")


def _operands(M, N, K, seed):
    A, _ = gemm_inputs.fp8_matrix(M, K, seed)
    B, _ = gemm_inputs.fp8_matrix(N, K, seed + 1)
    return A, B


def _same(x, y):
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


# scale pairs: ordinary values, a power-of-two pair, and one whose fp32
# product rounds (so the by-value and device products must round alike)
SCALES = [(0.37, 1.9), (0.25, 8.0), (1.0 / 3.0, 3.0000002)]


@pytest.mark.parametrize("schedule", ["interleave4", "pingpong8", "smalltile", "basic"])
def test_device_scales_match_by_value(schedule):
    M, N, K = 600, 520, 640   # edge tiles, several stages
    A, B = _operands(M, N, K, 101)
    Ad, Bd = A.view(torch.uint8).cuda(), B.view(torch.uint8).cuda()
    C0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C1 = torch.empty_like(C0)
    for sa, sb in SCALES:
        hk.hk_gemm_ex(FP8, Ad, Bd, C0, M, N, K, K, K, N, sa, sb, schedule=schedule)
        pa, pb = _dev(sa), _dev(sb)
        # both factors on the device (the by-value ones are then ignored), and
        # each alone with the other by value
        for kw, va, vb in (({"scale_a_dev": pa, "scale_b_dev": pb}, 5.0, 7.0),
                           ({"scale_a_dev": pa}, 5.0, sb),
                           ({"scale_b_dev": pb}, sa, 7.0)):
            C1.fill_(float("nan"))
            hk.hk_gemm_ex(FP8, Ad, Bd, C1, M, N, K, K, K, N, va, vb, schedule=schedule, **kw)
            torch.cuda.synchronize()
            same = _same(C0, C1)
            _say(schedule, (sa, sb), sorted(kw), "bit-identical to by-value:", same)
            assert same
    # the last pair against the oracle with the device values
    ref, S = oracle.gemm("fp8", gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(), M, N, K,
                         scale_a=float(np.float32(sa)), scale_b=float(np.float32(sb)))
    st = oracle.compare(_bits(C1), ref, S, rel_tol=RTOL)
    assert st["ok"], st


@pytest.mark.parametrize("layout_a,layout_b", [(0, 1), (1, 0), (1, 1)])
def test_device_scales_stored_transposed(layout_a, layout_b):
    """The 4-wave FP8 kernels for K-strided operands read the scales too."""
    M, N, K = 528, 608, 656
    A, B = _operands(M, N, K, 111)
    At = A.view(torch.uint8).t().contiguous() if layout_a else A.view(torch.uint8)
    Bt = B.view(torch.uint8).t().contiguous() if layout_b else B.view(torch.uint8)
    lda = M if layout_a else K
    ldb = N if layout_b else K
    Ad, Bd = At.cuda(), Bt.cuda()
    C0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C1 = torch.full_like(C0, float("nan"))
    sa, sb = 0.61, 1.37
    hk.hk_gemm_ex(FP8, Ad, Bd, C0, M, N, K, lda, ldb, N, sa, sb, layout_a=layout_a,
                  layout_b=layout_b)
    hk.hk_gemm_ex(FP8, Ad, Bd, C1, M, N, K, lda, ldb, N, 1.0, 1.0, layout_a=layout_a,
                  layout_b=layout_b, scale_a_dev=_dev(sa), scale_b_dev=_dev(sb))
    torch.cuda.synchronize()
    p = hk.hk_gemm_plan(FP8, Ad, Bd, C1, M, N, K, lda, ldb, N, layout_a=layout_a,
                        layout_b=layout_b)
    _say("layouts", (layout_a, layout_b), p["kernel_name"])
    assert p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4
    assert _same(C0, C1)


def test_non_finite_by_value_scale_replaced_by_a_pointer():
    """A by-value scale that a device pointer replaces is not checked."""
    M, N, K = 300, 260, 256
    A, B = _operands(M, N, K, 121)
    Ad, Bd = A.view(torch.uint8).cuda(), B.view(torch.uint8).cuda()
    C0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C1 = torch.empty_like(C0)
    hk.hk_gemm_ex(FP8, Ad, Bd, C0, M, N, K, K, K, N, 0.5, 2.5)
    hk.hk_gemm_ex(FP8, Ad, Bd, C1, M, N, K, K, K, N, float("nan"), 2.5, scale_a_dev=_dev(0.5))
    torch.cuda.synchronize()
    assert _same(C0, C1)


def test_device_scales_under_graph_replay():
    """A graph captured with device scales (and the no-alloc entry point with a
    repack, so two kernels) reads the scale values current at each replay."""
    M, N, K = 600, 700, 512
    ld = K + 16                   # 528-byte rows: the operands are repacked
    A = torch.empty(M, ld, dtype=torch.uint8, device="cuda")
    B = torch.empty(N, ld, dtype=torch.uint8, device="cuda")
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C)
    pa, pb = _dev(1.0), _dev(1.0)

    def fill(seed):
        A.copy_(gemm_inputs.fp8_matrix(M, ld, seed)[0].view(torch.uint8).cuda())
        B.copy_(gemm_inputs.fp8_matrix(N, ld, seed + 1)[0].view(torch.uint8).cuda())

    def call():
        hk.hk_gemm_ex_noalloc(FP8, A, B, C, M, N, K, ld, ld, N, 1.0, 1.0, repack="always",
                              scale_a_dev=pa, scale_b_dev=pb)

    fill(131)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep, (sa, sb) in enumerate([(0.75, 1.5), (3.0, 0.125), (0.37, 1.9)]):
        fill(140 + 2 * rep)
        pa.fill_(sa)
        pb.fill_(sb)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hk.hk_gemm_ex(FP8, A, B, C2, M, N, K, ld, ld, N, sa, sb, repack="never")
        torch.cuda.synchronize()
        same = _same(C, C2)
        _say("graph replay", rep, (sa, sb), "bit-identical to eager by-value:", same)
        assert same
    ref, S = oracle.gemm("fp8", gemm_inputs.bits(A.cpu()).ravel(), gemm_inputs.bits(B.cpu()).ravel(),
                         M, N, K, lda=ld, ldb=ld, scale_a=float(np.float32(sa)),
                         scale_b=float(np.float32(sb)))
    st = oracle.compare(_bits(C), ref, S, rel_tol=RTOL)
    assert st["ok"], st
