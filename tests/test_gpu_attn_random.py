"""Seeded random configurations of the attention forward against the oracle,
through the C ABI (hk.attention, which passes the tensors' strides).

Each case draws, from its own fixed seed: B (1-3), the key/value heads and the
grouping (query heads = key/value heads x 1, 2 or 4), N (biased towards the
64-key and 128-query block edges, up to about 1100), D (64 or 128), causal or
not, the softmax scale, the spread of the scores (values scaled by 1 or 3, so
that the running maximum moves and the lazy rescale runs), and the storage:
packed (B, H, N, D), (B, N, H, D) seen through a transpose, or rows padded
past D with NaN (O's padding then holds a sentinel that must survive).  O
must be within ulp_bf16(O_ref) + 2^-8 A of the oracle's matmul path and the
log-sum-exp within 1e-5 (1 + |lse|) + N 2^-24, as in the other attention
tests.
"""
import numpy as np
import pytest
import torch

import fp8_gemm_02_amd as hk
import gemm_inputs
import oracle
from oracle import matmul as oracle_matmul

RTOL = 2.0 ** -8
NCASES = 32
SENTINEL = 0x7BAD


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    hk.lib()
    torch.cuda.set_device(0)


def _say(*a):
    print("[gpu-attn-random]", *a, flush=True)


def _draw(seed):
    rng = np.random.default_rng(seed)
    c = {"B": int(rng.integers(1, 4)), "Hkv": int(rng.choice([1, 2, 4])),
         "group": int(rng.choice([1, 2, 4])), "D": int(rng.choice([64, 128])),
         "causal": bool(rng.integers(0, 2))}
    c["Hq"] = c["Hkv"] * c["group"]
    if rng.integers(0, 2):
        c["N"] = int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 383, 513]))
    else:
        c["N"] = int(rng.integers(1, 1100))
    c["scale"] = float(c["D"] ** -0.5) if rng.integers(0, 2) else float(rng.uniform(0.05, 0.3))
    c["spread"] = float(rng.choice([1.0, 3.0]))
    c["storage"] = str(rng.choice(["bhnd", "bnhd", "padded"]))
    return c


def _tensor(B, H, N, D, spread, seed):
    x = gemm_inputs.bf16_matrix(B * H * N, D, "normal", seed).float() * spread
    return x.to(torch.bfloat16).reshape(B, H, N, D)


def _lay_out(x, storage):
    """A device tensor with x's values in the chosen storage (a view when strided)."""
    B, H, N, D = x.shape
    if storage == "bhnd":
        return x.cuda()
    if storage == "bnhd":
        return x.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    # rows padded by 8 elements of NaN (token stride D + 8)
    buf = torch.full((B, H, N, D + 8), float("nan"), dtype=torch.bfloat16)
    buf[..., :D] = x
    return buf.cuda()[..., :D]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(NCASES))
def test_random_attention(gpu, case):
    c = _draw(7700 + case)
    B, Hq, Hkv, N, D = c["B"], c["Hq"], c["Hkv"], c["N"], c["D"]
    q = _tensor(B, Hq, N, D, c["spread"], 7800 + 3 * case)
    k = _tensor(B, Hkv, N, D, c["spread"], 7801 + 3 * case)
    v = _tensor(B, Hkv, N, D, 1.0, 7802 + 3 * case)
    _say(case, c)
    qd, kd, vd = (_lay_out(t, c["storage"]) for t in (q, k, v))
    if c["storage"] == "padded":
        obuf = torch.full((B, Hq, N, D + 8), 0, dtype=torch.int16, device="cuda")
        obuf.fill_(SENTINEL)
        out = obuf.view(torch.bfloat16)[..., :D]
    else:
        out = None
    O, L = hk.attention(qd, kd, vd, causal=c["causal"], scale=c["scale"], return_lse=True,
                        out=out)
    torch.cuda.synchronize()
    if c["storage"] == "padded":
        pad = obuf[..., D:].cpu().numpy().view(np.uint16)
        assert (pad == SENTINEL).all(), "O padding written"
    got = O.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, D)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16).ravel()
    ref, _, ref_lse, A = oracle_matmul.attention_by_matmul(bits(q), bits(k), bits(v), B, Hq, Hkv,
                                                           N, D, c["scale"], c["causal"])
    st = oracle.compare(got, ref, A, rel_tol=RTOL)
    lse = L.cpu().numpy().ravel()
    lbound = 1e-5 * (1 + np.abs(ref_lse)) + N * 2.0 ** -24
    lerr = np.abs(lse - ref_lse)
    _say(case, "ok" if st["ok"] else "FAIL", {k_: st[k_] for k_ in st if k_ != "ulp_hist"},
         "lse err/bound %.3g" % (lerr / lbound).max())
    assert st["ok"], (c, st)
    assert (lerr <= lbound).all(), (c, (lerr / lbound).max())


def test_the_attention_draws_cover_the_cases():
    """A CPU check of the fixed draws: both head dimensions, causal and not,
    grouped heads, every storage, N at block edges and N = 1."""
    cs = [_draw(7700 + i) for i in range(NCASES)]
    assert {c["D"] for c in cs} == {64, 128}
    assert {c["causal"] for c in cs} == {False, True}
    assert {c["storage"] for c in cs} == {"bhnd", "bnhd", "padded"}
    assert any(c["group"] > 1 for c in cs) and any(c["group"] == 1 for c in cs)
    assert any(c["N"] % 64 == 1 for c in cs) and any(c["N"] % 128 == 0 for c in cs)
    assert any(c["N"] == 1 for c in cs)
    assert any(c["spread"] > 1 for c in cs)
