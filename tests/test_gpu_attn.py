"""GPU parity of the attention forward (hk_attn_fwd_bf16 through the C ABI)
against the CPU oracle.

Acceptance rule, element by element: |O_gpu - O_ref| <= ulp_bf16(O_ref) +
2^-8 * A, with A = sum_j p_j |v_j| / sum_j p_j from the oracle.  The kernel
rounds the probabilities to bf16 (relative error at most 2^-9) before they
meet V, accumulates in fp32 and rounds the result once; 2^-8 * A covers the
first with a factor of two, the ulp term the final rounding.  The
log-sum-exp must lie within 1e-5 * (1 + |lse|) + N * 2^-24 of the oracle's
(fp32 sums of N terms).  Cases whose exact result survives fp32 (all-zero
queries over 2^k keys with integer values; one key dominating by more than
the fp32 exponent range) must match bit for bit.

Shapes cover one workgroup, ragged N (a partial query block and a partial
key block), N = 1, grouped-query heads, both head dimensions, causal and
non-causal, strided (B, N, H, D) storage with poisoned padding, more
workgroups than compute units, and the benchmark's workloads at full size
(sampled rows against the oracle's loop, every row against its matmul path).
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle
from oracle import matmul as oracle_matmul

pytestmark = pytest.mark.gpu

RTOL = 2.0 ** -8


def _say(*a):
    print("[gpu-attn]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(q, k, v, causal, scale, strides=None, lse=True):
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    O = torch.zeros((B, Hq, N, D), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    L = torch.zeros((B, Hq, N), dtype=torch.float32, device="cuda") if lse else None
    hk.hk_attn_fwd_bf16(q, k, v, O, L, B, Hq, Hkv, N, D, scale, causal, strides=strides)
    torch.cuda.synchronize()
    return O, L


def _check(q, k, v, causal, scale=None, exact=False, rows=None, tag=""):
    """q, k, v: CPU bf16 (B, H, N, D), packed."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    scale = D ** -0.5 if scale is None else scale
    O, L = _run(q.cuda(), k.cuda(), v.cuda(), causal, scale)
    got = _bits(O).reshape(-1, D)
    lse = L.cpu().numpy().ravel()
    ref, _, ref_lse, A = oracle.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(), B,
                                          Hq, Hkv, N, D, scale, causal, rows=rows)
    if rows is not None:
        got, lse = got[rows], lse[rows]
    st = oracle.compare(got, ref, A, exact=exact, rel_tol=RTOL)
    lbound = 1e-5 * (1 + np.abs(ref_lse)) + N * 2.0 ** -24
    lerr = np.abs(lse - ref_lse)
    _say(tag, (B, Hq, Hkv, N, D), "causal" if causal else "full", "exact" if exact else "tol",
         {k_: st[k_] for k_ in st if k_ != "ulp_hist"}, "lse err/bound %.3g" % (lerr / lbound).max())
    assert st["ok"], st
    assert (lerr <= lbound).all(), (lerr / lbound).max()


def _qkv(B, Hq, Hkv, N, D, seed, sd=1.0):
    return (gemm_inputs.bf16_matrix(B * Hq * N, D, "normal", seed).reshape(B, Hq, N, D) * sd,
            gemm_inputs.bf16_matrix(B * Hkv * N, D, "normal", seed + 1).reshape(B, Hkv, N, D) * sd,
            gemm_inputs.bf16_matrix(B * Hkv * N, D, "normal", seed + 2).reshape(B, Hkv, N, D))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 1, 1, 128, 128), (1, 1, 1, 128, 64),
                                          (2, 4, 2, 300, 128), (1, 3, 1, 1, 64),
                                          (1, 2, 1, 65, 128), (2, 2, 2, 777, 64),
                                          (1, 2, 2, 64, 128), (1, 4, 4, 1000, 128)])
def test_attn_full(B, Hq, Hkv, N, D, causal):
    q, k, v = _qkv(B, Hq, Hkv, N, D, 7 * N + D + Hq)
    _check(q, k, v, causal)


@pytest.mark.parametrize("D", [64, 128])
def test_attn_large_scores(D):
    """Scores with a spread of several hundred (sharp softmax): the running
    max and the rescaling of earlier blocks carry the result."""
    q, k, v = _qkv(1, 2, 1, 520, D, 33, sd=4.0)
    _check(q, k, v, False, scale=0.5)
    _check(q, k, v, True, scale=0.5)


@pytest.mark.parametrize("D", [64, 128])
def test_attn_zero_queries_exact(D):
    """All-zero queries over 256 keys with values in {-4..4}: every weight is
    exactly 1, so O is the exact mean of the value rows, rounded once."""
    B, H, N = 1, 2, 256
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    k = gemm_inputs.bf16_matrix(B * H * N, D, "normal", 3).reshape(B, H, N, D)
    v = gemm_inputs.bf16_matrix(B * H * N, D, "int4", 4).reshape(B, H, N, D)
    _check(q, k, v, False, exact=True)


def test_attn_dominant_key_exact():
    """Key 77 scores 2000 above every other key for every query: all other
    weights underflow to zero in fp32, so O is key 77's value row exactly."""
    B, H, N, D = 1, 1, 200, 128
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    q[..., 0] = 1.0
    k = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    k[0, 0, :, 0] = torch.linspace(-4, 4, N).to(torch.bfloat16)
    k[0, 0, 77, 0] = 2048.0
    v = gemm_inputs.bf16_matrix(N, D, "normal", 5).reshape(B, H, N, D)
    _check(q, k, v, False, scale=1.0, exact=True)
    O, _ = _run(q.cuda(), k.cuda(), v.cuda(), False, 1.0)
    assert np.array_equal(_bits(O)[0, 0], np.tile(_bits(v)[0, 0, 77], (N, 1)))


def test_attn_first_causal_row_is_v0():
    q, k, v = _qkv(1, 4, 2, 300, 128, 91)
    O, _ = _run(q.cuda(), k.cuda(), v.cuda(), True, 0.09)
    for h in range(4):
        assert np.array_equal(_bits(O)[0, h, 0], _bits(v)[0, h // 2, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_attn_strided_bnhd_poisoned(causal):
    """Q, K, V stored as (B, N, H, D) with padding between heads and tokens
    (NaN), O written into a padded (B, H, N, D) buffer whose padding must
    stay untouched."""
    B, Hq, Hkv, N, D = 2, 4, 2, 200, 64
    q, k, v = _qkv(B, Hq, Hkv, N, D, 55)

    def bnhd(x, pad_h, pad_t):
        Bx, H, Nx, Dx = x.shape
        sh, st = Dx + pad_h, H * (Dx + pad_h) + pad_t
        buf = torch.full((Bx * Nx * st,), 0x7FC0, dtype=torch.int16).view(torch.bfloat16)
        view = buf.as_strided((Bx, H, Nx, Dx), (Nx * st, sh, st, 1))
        view.copy_(x)
        return buf.cuda(), (Nx * st, sh, st)

    qb, sq = bnhd(q, 8, 16)
    kb, sk = bnhd(k, 0, 8)
    vb, sv = bnhd(v, 24, 0)
    so = (Hq * (N * D + 64), N * D + 64, D)
    Ob = torch.full((B * so[0],), 0x3F80, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    L = torch.zeros((B, Hq, N), dtype=torch.float32, device="cuda")
    hk.hk_attn_fwd_bf16(qb, kb, vb, Ob, L, B, Hq, Hkv, N, D, D ** -0.5, causal,
                        strides=[sq, sk, sv, so])
    torch.cuda.synchronize()
    O = Ob.as_strided((B, Hq, N, D), (so[0], so[1], so[2], 1))
    got = _bits(O).reshape(-1, D)
    ref, _, _, A = oracle.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(), B, Hq,
                                    Hkv, N, D, D ** -0.5, causal)
    st = oracle.compare(got, ref, A, rel_tol=RTOL)
    _say("strided", {k_: st[k_] for k_ in st if k_ != "ulp_hist"})
    assert st["ok"], st
    pad = _bits(Ob).reshape(B, Hq, -1)[:, :, N * D:]
    assert (pad == 0x3F80).all()


def test_attn_torch_views_and_no_lse():
    """hk.attention over a (B, N, H, D) tensor seen as (B, H, N, D), without
    the log-sum-exp output."""
    B, H, N, D = 2, 4, 256, 128
    q, k, v = _qkv(B, H, H, N, D, 61)
    qv = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    kv_ = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vv = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    O = hk.attention(qv, kv_, vv, causal=True)
    torch.cuda.synchronize()
    ref, _, _, A = oracle.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(), B, H,
                                    H, N, D, D ** -0.5, True)
    st = oracle.compare(_bits(O).reshape(-1, D), ref, A, rel_tol=RTOL)
    assert st["ok"], st


def test_attn_many_workgroups():
    """B * H * N / 128 = 512 workgroups, more than the compute units."""
    q, k, v = _qkv(4, 16, 4, 1024, 64, 71)
    rows = np.random.default_rng(1).integers(0, 4 * 16 * 1024, 3000)
    _check(q, k, v, True, rows=rows, tag="many")


@pytest.mark.parametrize("name", ["attn_d128_n4096", "attn_d128_n4096_causal", "attn_d64_n4096",
                                  "attn_gqa_d128_n8192_causal"])
def test_attn_full_size(name):
    """The benchmark's workloads as bench.py launches them: sampled rows
    (random plus the first and last rows of heads and query blocks) against
    the oracle's loop, then every row, O and LSE, against its matmul path."""
    w = gemm_inputs.ATTN_WORKLOADS[name]
    x = gemm_inputs.make_attn_inputs(w)
    rng = np.random.default_rng(7)
    nrow = w.B * w.Hq * w.N
    edge = [0, 1, 127, 128, w.N - 1, w.N - 128, nrow - 1, nrow - w.N]
    rows = np.concatenate([rng.integers(0, nrow, 400), edge])
    q, k, v = x["q"], x["k"], x["v"]
    O, L = _run(q.cuda(), k.cuda(), v.cuda(), w.causal, w.scale)
    got_all = _bits(O).reshape(-1, w.D)
    lse_all = L.cpu().numpy().ravel()
    got, lse = got_all[rows], lse_all[rows]
    del O, L
    ref, _, ref_lse, A = oracle.attention(_bits(q).ravel(), _bits(k).ravel(), _bits(v).ravel(),
                                          w.B, w.Hq, w.Hkv, w.N, w.D, w.scale, w.causal,
                                          rows=rows)
    st = oracle.compare(got, ref, A, rel_tol=RTOL)
    lbound = 1e-5 * (1 + np.abs(ref_lse)) + w.N * 2.0 ** -24
    _say(name, "sampled", rows.size, {k_: st[k_] for k_ in st if k_ != "ulp_hist"},
         "lse err/bound %.3g" % (np.abs(lse - ref_lse) / lbound).max())
    assert st["ok"], st
    assert (np.abs(lse - ref_lse) <= lbound).all()
    ref, _, ref_lse, A = oracle_matmul.attention_by_matmul(_bits(q).ravel(), _bits(k).ravel(),
                                                           _bits(v).ravel(), w.B, w.Hq, w.Hkv, w.N,
                                                           w.D, w.scale, w.causal)
    st = oracle.compare(got_all, ref, A, rel_tol=RTOL)
    lbound = 1e-5 * (1 + np.abs(ref_lse)) + w.N * 2.0 ** -24
    lratio = (np.abs(lse_all - ref_lse) / lbound).max()
    _say(name, "every row", {k_: st[k_] for k_ in st if k_ != "ulp_hist"},
         "lse err/bound %.3g" % lratio)
    assert st["ok"], st
    assert lratio <= 1.0


# The causal kernels are persistent: a grid of as many workgroups as the
# compute units hold (2 per unit at D = 128, 3 at D = 64) walks pairs of query
# blocks (the longest with the shortest; the middle block alone when their
# count is odd), prefetching each next tile's first key block during the
# current tile's last.  Shapes with more pairs than workgroups make some
# workgroups run several tiles in a row, with ragged N, an odd number of query
# blocks and grouped-query heads; compared in full.
@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(4, 48, 16, 600, 128), (3, 96, 32, 600, 64),
                                          (2, 40, 40, 1300, 128)])
def test_attn_causal_persistent_several_tiles_per_workgroup(B, Hq, Hkv, N, D):
    nqb = (N + 127) // 128
    units = B * Hq * ((nqb + 1) // 2)
    slots = (3 if D == 64 else 2) * 256
    assert units > slots or B * Hq * nqb > slots  # several tiles in a row somewhere
    q, k, v = _qkv(B, Hq, Hkv, N, D, 300 + D)
    _check(q, k, v, True, tag="persistent causal, %d pairs" % units)
