"""hk_gemm_ex_noalloc: the same product as hk_gemm_ex with a workspace, with
the repack workspace taken from the library's own device array.

Called through the C ABI and compared bit for bit with hk_gemm_ex given a
torch-allocated workspace (the copies change neither the tile walk nor the K
order, so the results are identical), on two calls in a row, the second with
a smaller input, so that the second runs over what the first left in the
array.  Also: a call that would need more than the array is refused with
nothing written, and a caller workspace is refused.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _say(*a):
    print("[no-alloc]", *a, flush=True)


def _operands(dtype, M, N, K, ld, seed):
    if dtype == "bf16":
        return (gemm_inputs.bf16_matrix(M, ld, "uniform", seed).cuda(),
                gemm_inputs.bf16_matrix(N, ld, "uniform", seed + 1).cuda(), 1.0, 1.0)
    A, sa = gemm_inputs.fp8_matrix(M, ld, seed)
    B, sb = gemm_inputs.fp8_matrix(N, ld, seed + 1)
    return A.cuda(), B.cuda(), sa, sb


def _call_pair(dtype, M, N, K, ld, seed, repack):
    dt = hk.HK_DTYPE_BF16 if dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
    A, B, sa, sb = _operands(dtype, M, N, K, ld, seed)
    need = hk.hk_gemm_workspace_size(dt, A, B, A, M, N, K, ld, ld, N, repack=repack)
    assert 0 < need <= hk.HK_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    C_ex = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    C_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    hk.hk_gemm_ex(dt, A, B, C_ex, M, N, K, ld, ld, N, sa, sb, workspace=ws, repack=repack)
    # through the C ABI directly, as a caller without torch would
    o = hk.GemmOpts()
    o.repack = hk.REPACKS[repack]
    st = hk.lib().hk_gemm_ex_noalloc(dt, ctypes.c_void_p(A.data_ptr()),
                                     ctypes.c_void_p(B.data_ptr()),
                                     ctypes.c_void_p(C_na.data_ptr()), M, N, K, ld, ld, N,
                                     ctypes.c_float(sa), ctypes.c_float(sb), ctypes.byref(o),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == hk.HK_SUCCESS, hk.status_string(st)
    torch.cuda.synchronize()
    same = torch.equal(C_ex.view(torch.int16), C_na.view(torch.int16))
    # and the oracle, on a sample, for the record
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M, 500)
    cols = rng.integers(0, N, 500)
    got = C_na[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()]
    got = got.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, S = oracle.gemm_sampled(dtype, gemm_inputs.bits(A.cpu()).ravel(),
                                 gemm_inputs.bits(B.cpu()).ravel(), M, N, K, rows, cols,
                                 lda=ld, ldb=ld, scale_a=sa, scale_b=sb)
    cmp = oracle.compare(got, ref, S, rel_tol=1e-4)
    _say(dtype, (M, N, K, ld), repack, "scratch bytes", need, "identical:", same,
         {k: cmp[k] for k in cmp if k != "ulp_hist"})
    assert same and cmp["ok"]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_ex_twice_second_smaller(dtype):
    # rows of ld elements straddle cache lines, so both operands are copied
    if dtype == "bf16":
        _call_pair(dtype, 2048, 3072, 2056, 2056, 101, "always")
        _call_pair(dtype, 700, 900, 1032, 1040, 103, "always")
    else:
        _call_pair(dtype, 2048, 3072, 2064, 2064, 105, "always")
        _call_pair(dtype, 700, 900, 1040, 1056, 107, "always")


def test_noalloc_auto_at_a_size_that_pays():
    # M N >= 4096 (M + N): AUTO copies both operands (8208-byte rows to 9 KiB)
    _call_pair("bf16", 8192, 8192, 4104, 4104, 109, "auto")


def test_noalloc_refuses_what_does_not_fit_and_caller_workspaces():
    M, N, K = 8191, 28670, 8200  # needs 642 MB of copies
    fake = 1 << 20
    need = hk.hk_gemm_workspace_size(hk.HK_DTYPE_BF16, fake, fake, fake, M, N, K, K, K, N)
    assert need > hk.HK_NOALLOC_SCRATCH_BYTES
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    st = hk.hk_gemm_ex_noalloc(hk.HK_DTYPE_BF16, A, B, C, M, N, K, K, K, N, raise_on_error=False)
    torch.cuda.synchronize()
    assert st == hk.HK_ERROR_NOT_SUPPORTED
    assert bool((C == 3.0).all())  # nothing was enqueued
    # without copies it runs on the operands as given
    st = hk.hk_gemm_ex_noalloc(hk.HK_DTYPE_BF16, A, B, C, M, N, K, K, K, N, repack="never",
                               raise_on_error=False)
    torch.cuda.synchronize()
    assert st == hk.HK_SUCCESS and bool((C == 0).all())
    # a caller workspace is the other entry point's business
    o = hk.GemmOpts()
    o.workspace, o.workspace_bytes = fake, 4096
    st = hk.lib().hk_gemm_ex_noalloc(0, fake, fake, fake, 64, 64, 64, 64, 64, 64,
                                     ctypes.c_float(1), ctypes.c_float(1), ctypes.byref(o), None)
    assert st == hk.HK_ERROR_INVALID_VALUE
