"""The entry points under HIP graph capture (torch.cuda.graph), through the C ABI.

Each call enqueues only kernel launches on the caller's stream (no memset, no
allocation, no synchronisation), so it can be captured.  Every test captures
one call, then replays the graph several times.  Between replays the program
does its own eager work: it writes fresh values into the inputs in place and
poisons the output.  Each replay must then equal, bit for bit, an eager call
on the same inputs.  That shows the graph reads the buffers' current contents
and rewrites every output element.  One replay is also checked against the
oracle.

Covered: hk_gemm_bf16 on a ragged shape, hk_gemm_ex_noalloc repacking
operands whose rows straddle cache lines (two kernels in the graph, the
workspace in the library's own array), and the causal attention forward.
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu
RTOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _say(*a):
    print("[gpu-graph]", *a, flush=True)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _capture(fn):
    """Run fn once eagerly, then capture it into a graph."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _refill(t, seed):
    """New bf16 values in place (eager work between replays)."""
    src = gemm_inputs.bf16_matrix(t.numel() // t.shape[-1], t.shape[-1], "uniform", seed)
    t.copy_(src.reshape(t.shape).cuda())


def test_gemm_bf16_replays():
    M, N, K = 1000, 777, 520   # ragged edges and a K tail
    A = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C)
    _refill(A, 1)
    _refill(B, 2)
    g = _capture(lambda: hk.hk_gemm_bf16(A, B, C, M, N, K, K, K, N))
    for rep in range(4):
        _refill(A, 10 + rep)
        _refill(B, 20 + rep)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hk.hk_gemm_bf16(A, B, C2, M, N, K, K, K, N)
        torch.cuda.synchronize()
        same = torch.equal(C.view(torch.int16), C2.view(torch.int16))
        _say("hk_gemm_bf16 replay", rep, "bit-identical to eager:", same)
        assert same
    ref, S = oracle.gemm("bf16", gemm_inputs.bits(A.cpu()).ravel(), gemm_inputs.bits(B.cpu()).ravel(),
                         M, N, K)
    st = oracle.compare(_bits(C), ref, S, rel_tol=RTOL)
    assert st["ok"], st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gemm_noalloc_repack_replays(dtype):
    """Rows that straddle cache lines, REPACK_ALWAYS: the graph holds the copy
    launch and the product launch, with the copies in the library's array."""
    M, N, K = 600, 700, 512
    if dtype == "bf16":
        ld, dt = K + 8, hk.HK_DTYPE_BF16     # 1040-byte rows
        A = torch.empty(M, ld, dtype=torch.bfloat16, device="cuda")
        B = torch.empty(N, ld, dtype=torch.bfloat16, device="cuda")
        sa = sb = 1.0

        def fill(seed):
            _refill(A, seed)
            _refill(B, seed + 1)
    else:
        ld, dt = K + 16, hk.HK_DTYPE_FP8_E4M3   # 528-byte rows
        A = torch.empty(M, ld, dtype=torch.uint8, device="cuda")
        B = torch.empty(N, ld, dtype=torch.uint8, device="cuda")
        sa, sb = 0.5, 2.0

        def fill(seed):
            A.copy_(gemm_inputs.fp8_matrix(M, ld, seed)[0].view(torch.uint8).cuda())
            B.copy_(gemm_inputs.fp8_matrix(N, ld, seed + 1)[0].view(torch.uint8).cuda())
    assert (ld * A.element_size()) % 128 != 0
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C)
    need = hk.hk_gemm_workspace_size(dt, A, B, C, M, N, K, ld, ld, N, repack="always")
    assert 0 < need <= hk.HK_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    fill(31)
    g = _capture(lambda: hk.hk_gemm_ex_noalloc(dt, A, B, C, M, N, K, ld, ld, N, sa, sb,
                                               repack="always"))
    for rep in range(3):
        fill(40 + 2 * rep)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hk.hk_gemm_ex(dt, A, B, C2, M, N, K, ld, ld, N, sa, sb, repack="always", workspace=ws)
        torch.cuda.synchronize()
        same = torch.equal(C.view(torch.int16), C2.view(torch.int16))
        _say("noalloc", dtype, "replay", rep, "bit-identical to eager with a workspace:", same)
        assert same
    ref, S = oracle.gemm(dtype, gemm_inputs.bits(A.cpu()).ravel(), gemm_inputs.bits(B.cpu()).ravel(),
                         M, N, K, lda=ld, ldb=ld, scale_a=sa, scale_b=sb)
    st = oracle.compare(_bits(C), ref, S, rel_tol=RTOL)
    assert st["ok"], st


def test_attention_causal_replays():
    Bn, Hq, Hkv, N, D = 2, 4, 2, 300, 128
    q = torch.empty(Bn, Hq, N, D, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(Bn, Hkv, N, D, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(Bn, Hkv, N, D, dtype=torch.bfloat16, device="cuda")
    O = torch.empty_like(q)
    O2 = torch.empty_like(q)
    L = torch.empty(Bn, Hq, N, dtype=torch.float32, device="cuda")
    L2 = torch.empty_like(L)
    scale = D ** -0.5
    for t, sd in ((q, 3), (k, 4), (v, 5)):
        _refill(t, sd)
    g = _capture(lambda: hk.hk_attn_fwd_bf16(q, k, v, O, L, Bn, Hq, Hkv, N, D, scale, True))
    for rep in range(3):
        for t, sd in ((q, 50 + rep), (k, 60 + rep), (v, 70 + rep)):
            _refill(t, sd)
        O.fill_(float("nan"))
        L.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        hk.hk_attn_fwd_bf16(q, k, v, O2, L2, Bn, Hq, Hkv, N, D, scale, True)
        torch.cuda.synchronize()
        same = torch.equal(O.view(torch.int16), O2.view(torch.int16)) and torch.equal(L, L2)
        _say("attention replay", rep, "bit-identical to eager:", same)
        assert same
    ref, _, ref_lse, A = oracle.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(),
                                          Bn, Hq, Hkv, N, D, scale, True)
    st = oracle.compare(_bits(O).reshape(-1, D), ref, A, rel_tol=2.0 ** -8)
    assert st["ok"], st
    lbound = 1e-5 * (1 + np.abs(ref_lse)) + N * 2.0 ** -24
    assert (np.abs(L.cpu().numpy().ravel() - ref_lse) <= lbound).all()
