"""GPU parity of the MXFP8 path (hk_gemm_mxfp8 through the C ABI) against the
CPU oracle's MXFP8 product.

Same acceptance rule as the other parity tests: bit-exact for integer-valued
elements (with scales 2^-1, 2^0, 2^1, whose sums stay exact in fp32),
otherwise |C_gpu - C_ref| <= ulp_bf16(C_ref) + 1e-4 * S.  Shapes span several
tiles, ragged M and N, K that is a multiple of 32 but not of a stage (128),
single-block K, padded strides with poisoned padding (NaN elements and NaN
scales), more tiles than compute units, and the full 8192^3 workload in the
benchmark's launch configuration (sampled entries).
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


def _say(*a):
    print("[gpu-mxfp8]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(A, B, SA, SB, M, N, K, lda, ldb, ldsa, ldsb, ldc=None):
    ldc = ldc or N
    C = torch.zeros((max(M, 1), ldc), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    hk.hk_gemm_mxfp8(A.cuda(), B.cuda(), C, M, N, K, lda, ldb, ldc, SA.cuda(), SB.cuda(), ldsa,
                     ldsb)
    torch.cuda.synchronize()
    return _bits16(C)[:M, :N]


def _inputs(M, N, K, seed, integer):
    A, SA = gemm_inputs.mxfp8_matrix(M, K, seed, integer)
    B, SB = gemm_inputs.mxfp8_matrix(N, K, seed + 1, integer)
    return A, B, SA, SB


def _pad_cols(t, ld, fill):
    """Copy a (rows, cols) uint8 tensor into rows of ld bytes, the rest `fill`."""
    rows, cols = t.shape
    out = torch.full((rows, ld), fill, dtype=torch.uint8)
    out[:, :cols] = t
    return out


def _check(A, B, SA, SB, M, N, K, exact, lda=None, ldb=None, ldsa=None, ldsb=None):
    nb = K // 32
    # the kernel reads scales as 16-byte rows: pad the packed arrays to a
    # multiple of 16 bytes (255 = NaN in the padding, which must never be used)
    ldsa = ldsa or ((nb + 15) // 16) * 16
    ldsb = ldsb or ((nb + 15) // 16) * 16
    lda = lda or K
    ldb = ldb or K
    Ap = _pad_cols(A, lda, 0x7F) if lda != K else A
    Bp = _pad_cols(B, ldb, 0x7F) if ldb != K else B
    SAp = _pad_cols(SA, ldsa, 255)
    SBp = _pad_cols(SB, ldsb, 255)
    got = _run(Ap, Bp, SAp, SBp, M, N, K, lda, ldb, ldsa, ldsb)
    ref, S = oracle.gemm_mx(Ap.numpy().ravel(), Bp.numpy().ravel(), SAp.numpy().ravel(),
                            SBp.numpy().ravel(), M, N, K, lda=lda, ldb=ldb, ldsa=ldsa, ldsb=ldsb)
    st = oracle.compare(got, ref, S, exact=exact, rel_tol=RTOL)
    _say((M, N, K), "exact" if exact else "tol", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    return st


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (520, 600, 640), (300, 1, 160), (33, 513, 32),
                                   (777, 1029, 512), (257, 300, 96), (64, 64, 4128)])
@pytest.mark.parametrize("integer", [True, False])
def test_mxfp8_full(M, N, K, integer):
    A, B, SA, SB = _inputs(M, N, K, 7 * M + N + K, integer)
    _check(A, B, SA, SB, M, N, K, exact=integer)


def test_mxfp8_padded_strides_poisoned():
    M, N, K = 300, 260, 384
    A, B, SA, SB = _inputs(M, N, K, 91, False)
    _check(A, B, SA, SB, M, N, K, exact=False, lda=K + 48, ldb=K + 16, ldsa=32, ldsb=48)


def test_mxfp8_wide_scale_range():
    """Scale bytes across 2^-40 .. 2^40 per block: each block's contribution is
    weighted independently, so a wrong block-to-lane pairing shows."""
    M, N, K = 256, 256, 512
    A, B, _, _ = _inputs(M, N, K, 17, False)
    g = torch.Generator().manual_seed(18)
    SA = torch.randint(87, 168, (M, K // 32), generator=g).to(torch.uint8)
    SB = torch.randint(87, 168, (N, K // 32), generator=g).to(torch.uint8)
    _check(A, B, SA, SB, M, N, K, exact=False)


def test_mxfp8_persistent_tile_walk():
    M, N, K = 4359, 4352, 640  # 306 tiles > 256 compute units; 5 stages (odd)
    A, B, SA, SB = _inputs(M, N, K, 23, True)
    _check(A, B, SA, SB, M, N, K, exact=True)


def test_mxfp8_full_size():
    """The 8192^3 workload exactly as the benchmark launches it (packed
    scales, ld = K / 32 = 256), checked on sampled entries with the oracle's
    loop and on every element with its matmul path."""
    w = gemm_inputs.WORKLOADS["mxfp8_8192"]
    x = gemm_inputs.make_inputs(w)
    nb = w.K // 32
    got = _run(x["A"], x["B"], x["SA"], x["SB"], w.M, w.N, w.K, w.K, w.K, nb, nb)
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.integers(0, w.M, 400), [0, w.M - 1, 255, 256, 4095]])
    cols = np.concatenate([rng.integers(0, w.N, 400), [w.N - 1, 0, 256, 255, 4096]])
    c, s = oracle.gemm_mx_sampled(gemm_inputs.bits(x["A"]).ravel(), gemm_inputs.bits(x["B"]).ravel(),
                                  x["SA"].numpy().ravel(), x["SB"].numpy().ravel(), w.M, w.N, w.K,
                                  rows, cols)
    st = oracle.compare(got[rows, cols], c, s, rel_tol=RTOL)
    _say("mxfp8_8192 sampled", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st
    ref, S = oracle_matmul.gemm_mx_by_matmul(gemm_inputs.bits(x["A"]), gemm_inputs.bits(x["B"]),
                                             x["SA"].numpy(), x["SB"].numpy(), w.M, w.N, w.K)
    st = oracle.compare(got, ref, S, rel_tol=RTOL)
    _say("mxfp8_8192 every element", {k: st[k] for k in st if k != "ulp_hist"})
    assert st["ok"], st


def test_mxfp8_zero_k_and_empty():
    C = torch.full((4, 4), 7.0, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(16, dtype=torch.uint8, device="cuda")
    hk.hk_gemm_mxfp8(z, z, C, 4, 4, 0, 16, 16, 4, z, z, 16, 16)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    hk.hk_gemm_mxfp8(z, z, C, 0, 4, 32, 32, 32, 4, z, z, 16, 16)


def test_mxfp8_nan_scale_matches_the_oracle():
    """E8M0 255 is NaN (OCP MX): a block with that scale poisons its row of C
    (scale of A) or its column (scale of B), on the GPU as in the oracle."""
    M, N, K = 64, 64, 256
    A, B, SA, SB = _inputs(M, N, K, 41, False)
    SA = SA.clone()
    SB = SB.clone()
    SA[5, 3] = 255
    SB[9, 0] = 255
    SAp, SBp = _pad_cols(SA, 16, 127), _pad_cols(SB, 16, 127)
    got = _run(A, B, SAp, SBp, M, N, K, K, K, 16, 16)
    ref, S = oracle.gemm_mx(gemm_inputs.bits(A).ravel(), gemm_inputs.bits(B).ravel(),
                            SAp.numpy().ravel(), SBp.numpy().ravel(), M, N, K, ldsa=16, ldsb=16)
    gnan = np.isnan(oracle.bf16_to_f64(got))
    rnan = np.isnan(oracle.bf16_to_f64(ref))
    assert rnan.sum() == M + N - 1
    assert np.array_equal(gnan, rnan)
    st = oracle.compare(np.where(rnan, 0, got), np.where(rnan, 0, ref), np.where(rnan, 0, S),
                        rel_tol=RTOL)
    assert st["ok"], st
