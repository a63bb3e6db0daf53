"""Seeded random configurations of hk_gemm_ex against the oracle, through the C ABI.

Each case draws, from its own fixed seed: the dtype (BF16 or FP8 E4M3), M, N
and K (1 to about 1500, with a bias towards tile and chunk edges), each
operand's layout (K-contiguous or K-strided) and row padding, the padding of
C's rows, the grid order, a schedule (AUTO, BASIC, or a fast schedule when the
documented fast-path conditions hold for the drawn case), and for FP8 whether
each scale comes by value or from device memory.  Padding is poisoned (NaN
operands, a sentinel in C) so that any read or write outside the logical
matrices shows.  Half the cases are integer-valued and must match bit for
bit; the others are checked with the acceptance rule
|C_gpu - C_ref| <= ulp_bf16(C_ref) + 1e-4 S, against the oracle's matmul path.
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle
from oracle import matmul as oracle_matmul

RTOL = 1e-4
SENTINEL = 0x7BAD
NCASES = 96


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _say(*a):
    print("[gpu-random]", *a, flush=True)


def _dim(rng, chunk):
    """A size biased towards edges: tile and chunk multiples, +-1 around them, or any."""
    kind = rng.integers(0, 4)
    if kind == 0:
        return int(rng.integers(1, 1500))
    if kind == 1:
        return int(rng.choice([1, 2, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65]))
    base = int(rng.choice([128, 256, 512, 768, 1024, 1280]))
    return max(1, base + int(rng.choice([-chunk, -1, 0, 1, chunk])))


def _draw(seed):
    rng = np.random.default_rng(seed)
    c = {"dtype": "bf16" if rng.integers(0, 2) == 0 else "fp8"}
    chunk = 8 if c["dtype"] == "bf16" else 16
    c["M"], c["N"], c["K"] = _dim(rng, chunk), _dim(rng, chunk), _dim(rng, chunk)
    c["integer"] = bool(rng.integers(0, 2))
    c["layout_a"], c["layout_b"] = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    # row padding: none, a whole number of chunks, or odd
    pads = [0, chunk, 3 * chunk, 1, 5]
    c["pad_a"], c["pad_b"] = int(rng.choice(pads)), int(rng.choice(pads))
    if rng.integers(0, 3) > 0:
        # two draws in three meet the fast-path conditions: the sizes the
        # stored rows run along, and the padding, in whole chunks
        up = lambda x: (x + chunk - 1) // chunk * chunk
        c["K"] = up(c["K"])
        if c["layout_a"]:
            c["M"] = up(c["M"])
        if c["layout_b"]:
            c["N"] = up(c["N"])
        c["pad_a"], c["pad_b"] = (int(rng.choice([0, chunk, 3 * chunk])) for _ in range(2))
    c["pad_c"] = int(rng.choice([0, 2, 8, 3]))
    c["grid_order"] = str(rng.choice(["auto", "row_major", "xcd"]))
    c["scale_dev"] = str(rng.choice(["none", "a", "b", "both"])) if c["dtype"] == "fp8" else "none"
    # the documented fast-path conditions for this case
    la = c["M"] if c["layout_a"] else c["K"]   # elements per stored row before padding
    lb = c["N"] if c["layout_b"] else c["K"]
    lda, ldb = la + c["pad_a"], lb + c["pad_b"]
    trans = c["layout_a"] or c["layout_b"]
    a_ok = lda % chunk == 0 and (c["M"] % chunk == 0 if c["layout_a"] else c["K"] % chunk == 0)
    b_ok = ldb % chunk == 0 and (c["N"] % chunk == 0 if c["layout_b"] else c["K"] % chunk == 0)
    fast = a_ok and b_ok
    choices = ["auto", "basic"]
    if fast:
        choices += ["interleave4"] * 2 if trans else ["interleave4", "pingpong8", "smalltile"]
        if not trans and c["dtype"] == "bf16":
            choices += ["interleave8", "producer_consumer"]
    c["schedule"] = str(rng.choice(choices))
    c["lda"], c["ldb"], c["ldc"] = lda, ldb, c["N"] + c["pad_c"]
    c["fast"] = fast
    return c


def _operand(dtype, rows, K, integer, seed):
    """Logical rows x K values: (bf16 tensor or e4m3 bytes, scale)."""
    if dtype == "bf16":
        return gemm_inputs.bf16_matrix(rows, K, "int4" if integer else "normal", seed), 1.0
    return gemm_inputs.fp8_matrix(rows, K, seed, integer=integer)


def _store(X, ld, strided, poison):
    """Lay the logical rows x K matrix X out as the GPU reads it, padding poisoned."""
    Y = X.t() if strided else X
    out = torch.full((Y.shape[0], ld), 0, dtype=X.dtype)
    out.view(torch.uint8 if X.dtype == torch.uint8 else torch.int16).fill_(poison)
    out[:, :Y.shape[1]] = Y
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(NCASES))
def test_random_config(gpu, case):
    c = _draw(9100 + case)
    dtype, M, N, K = c["dtype"], c["M"], c["N"], c["K"]
    A, sa = _operand(dtype, M, K, c["integer"], 9300 + 2 * case)
    B, sb = _operand(dtype, N, K, c["integer"], 9301 + 2 * case)
    if dtype == "fp8" and c["integer"]:
        sa, sb = 0.5, 4.0  # powers of two keep the scaled integer sums exact
    poison = 0x7FC0 if dtype == "bf16" else 0x7F   # NaN in bf16 / e4m3fn
    As = _store(A, c["lda"], c["layout_a"], poison)
    Bs = _store(B, c["ldb"], c["layout_b"], poison)
    _say(case, c)
    dt = hk.HK_DTYPE_BF16 if dtype == "bf16" else hk.HK_DTYPE_FP8_E4M3
    Cbuf = torch.full((M * c["ldc"],), SENTINEL, dtype=torch.int16, device="cuda")
    kw = {}
    va, vb = sa, sb
    if c["scale_dev"] in ("a", "both"):
        kw["scale_a_dev"] = torch.tensor([sa], dtype=torch.float32, device="cuda")
        va = 3.0  # ignored
    if c["scale_dev"] in ("b", "both"):
        kw["scale_b_dev"] = torch.tensor([sb], dtype=torch.float32, device="cuda")
        vb = 5.0  # ignored
    hk.hk_gemm_ex(dt, As.cuda(), Bs.cuda(), Cbuf, M, N, K, c["lda"], c["ldb"], c["ldc"], va, vb,
                  schedule=c["schedule"], grid_order=c["grid_order"], layout_a=c["layout_a"],
                  layout_b=c["layout_b"], **kw)
    torch.cuda.synchronize()
    allc = Cbuf.cpu().numpy().view(np.uint16).reshape(M, c["ldc"])
    assert (allc[:, N:] == SENTINEL).all(), "C padding written"
    ref, S = oracle_matmul.gemm_by_matmul(dtype, gemm_inputs.bits(A).ravel(),
                                          gemm_inputs.bits(B).ravel(), M, N, K,
                                          scale_a=float(np.float32(sa)),
                                          scale_b=float(np.float32(sb)))
    st = oracle.compare(allc[:, :N], ref, S, exact=c["integer"], rel_tol=RTOL)
    _say(case, "ok" if st["ok"] else "FAIL", {k: v for k, v in st.items() if k != "ulp_hist"})
    assert st["ok"], (c, st)


def test_the_draws_cover_every_schedule_and_layout():
    """The fixed seeds reach every schedule, both layouts of each operand,
    padded and odd strides, and device scales (a CPU check of the draws, so
    that a change of seeds cannot silently narrow the coverage)."""
    cs = [_draw(9100 + i) for i in range(NCASES)]
    assert {c["schedule"] for c in cs} >= {"auto", "basic", "interleave4", "pingpong8",
                                            "smalltile"}
    assert {(c["layout_a"], c["layout_b"]) for c in cs} == {(0, 0), (0, 1), (1, 0), (1, 1)}
    assert any(c["layout_a"] or c["layout_b"] for c in cs if c["schedule"] == "interleave4")
    assert {c["scale_dev"] for c in cs if c["dtype"] == "fp8"} == {"none", "a", "b", "both"}
    assert any(not c["fast"] for c in cs) and any(c["fast"] for c in cs)
    assert {c["dtype"] for c in cs} == {"bf16", "fp8"}
    assert any(c["integer"] for c in cs) and any(not c["integer"] for c in cs)
