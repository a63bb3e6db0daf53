"""Seeded synthetic inputs for C = A * B^T, shared by the tests, the smoke check
and the benchmark.

This module holds the workload definitions and random draws only; it contains
none of the product's arithmetic and imports neither the GPU library nor the
oracle.  Everything is drawn on the CPU with ``torch.Generator`` so that any
machine reproduces the same bytes for a given seed.

Workloads (M x N x K, operands K-contiguous, A is M x K, B is N x K):

* ``bf16_256``        256^3, Uniform[-1, 1] rounded once to bf16, plus an
                      integer-valued variant with entries in {-4..4};
* ``bf16_4096``       4096^3, Normal(0, 1);
* ``bf16_8192``       8192^3, Normal(0, 1) * 0.02 (the headline shape);
* ``bf16_mlp``        8192 x 28672 x 8192, Normal(0, 1) * 0.02 (tokens x FFN
                      width x model width);
* ``bf16_mlp_ragged`` 8191 x 28670 x 8200, same distribution (odd M, N not a
                      multiple of the tile, K tail of 8);
* ``fp8_8192``        8192^3, Normal(0, 1) scaled per tensor so that
                      max |x| = 448, rounded to OCP e4m3, with fp32 scales;
* ``mxfp8_8192``      8192^3, Normal(0, 1) quantised to MXFP8: per block of 32
                      K-values of a row, shared scale 2^(floor(log2 amax) - 8)
                      as an E8M0 byte, elements x / scale clamped to +-448 and
                      rounded to e4m3 (the conversion of the OCP MX v1.0
                      specification);
* ``bf16_mlp_shard8`` 8192 x 3584 x 8192: one GPU's share of the MLP shape
                      split eight ways along N;
* ``bf16_8192_bkn``   the bf16_8192 matrices with B stored K x N (C = A B);
* ``bf16_8192_akm_bkn`` the same with A stored K x M as well (C = A^T B with
                      the stored arrays);
* ``bf16_8192_akm``   the bf16_8192 matrices with A stored K x M only.
* ``fp8_8192_bkn``, ``fp8_8192_akm_bkn`` the fp8_8192 matrices with B (and A)
  stored K-strided.

Stored operands: a workload's layout_a / layout_b say how A and B sit in
memory (0: rows of K, A as M x K and B as N x K; 1: A as K x M, B as K x N).
make_inputs returns the logical M x K and N x K matrices, whatever the layout;
stored() gives the arrays as the layout stores them.

Seeds: workload index c gives A seed 1000c+1 and B seed 1000c+2; the integer
variant adds 10.

Attention workloads (ATTN_WORKLOADS, make_attn_inputs) draw Q, K and V the
same way, with seeds 1000c+1, +2, +3.
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    M: int
    N: int
    K: int
    dtype: str   # "bf16", "fp8" or "mxfp8"
    dist: str    # "uniform", "normal", "normal002", "int4", "fp8_normal"
    layout_a: int = 0  # 1: A stored K x M
    layout_b: int = 0  # 1: B stored K x N

    @property
    def lda(self) -> int:
        return self.M if self.layout_a else self.K

    @property
    def ldb(self) -> int:
        return self.N if self.layout_b else self.K

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 1

    @property
    def algorithmic_bytes(self) -> int:
        """Read each input once (with its block scales for MXFP8), write C (bf16) once."""
        scales = (self.M + self.N) * ((self.K + 31) // 32) if self.dtype == "mxfp8" else 0
        return (self.M + self.N) * self.K * self.in_bytes + scales + 2 * self.M * self.N

    def seeds(self, integer: bool = False):
        base = 1000 * self.index + (10 if integer else 0)
        return base + 1, base + 2


WORKLOADS = {
    w.name: w for w in [
        Workload("bf16_256", 0, 256, 256, 256, "bf16", "uniform"),
        Workload("bf16_4096", 1, 4096, 4096, 4096, "bf16", "normal"),
        Workload("bf16_8192", 2, 8192, 8192, 8192, "bf16", "normal002"),
        Workload("bf16_mlp", 3, 8192, 28672, 8192, "bf16", "normal002"),
        Workload("bf16_mlp_ragged", 3, 8191, 28670, 8200, "bf16", "normal002"),
        Workload("fp8_8192", 4, 8192, 8192, 8192, "fp8", "fp8_normal"),
        # one GPU's share of the MLP shape split over 8 GPUs along N (448
        # tiles of 256 x 256: 1.75 windows of 256 co-resident workgroups)
        Workload("bf16_mlp_shard8", 3, 8192, 3584, 8192, "bf16", "normal002"),
        Workload("mxfp8_8192", 5, 8192, 8192, 8192, "mxfp8", "mx_normal"),
        Workload("bf16_8192_bkn", 2, 8192, 8192, 8192, "bf16", "normal002", 0, 1),
        Workload("bf16_8192_akm_bkn", 2, 8192, 8192, 8192, "bf16", "normal002", 1, 1),
        Workload("bf16_8192_akm", 2, 8192, 8192, 8192, "bf16", "normal002", 1, 0),
        Workload("fp8_8192_bkn", 4, 8192, 8192, 8192, "fp8", "fp8_normal", 0, 1),
        Workload("fp8_8192_akm_bkn", 4, 8192, 8192, 8192, "fp8", "fp8_normal", 1, 1),
    ]
}


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """Attention forward: Q is B x Hq x N x D, K and V are B x Hkv x N x D
    (packed, D contiguous), entries Normal(0, 1) rounded once to bf16,
    softmax scale 1/sqrt(D)."""
    name: str
    index: int
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    causal: bool

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    @property
    def pairs(self) -> int:
        """(query, key) pairs the mask leaves visible, per head."""
        return self.N * (self.N + 1) // 2 if self.causal else self.N * self.N

    @property
    def flops(self) -> float:
        """Two products of 2 * D FLOP per visible (query, key) pair."""
        return 4.0 * self.B * self.Hq * self.pairs * self.D

    @property
    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O (bf16) and the fp32 log-sum-exp written once."""
        reads = 2 * self.B * (self.Hq + 2 * self.Hkv) * self.N * self.D
        return reads + 2 * self.B * self.Hq * self.N * self.D + 4 * self.B * self.Hq * self.N


# Sizes: the pages give none ("several head dimensions and sequence
# lengths"); these are 16K tokens per launch at sequence length 4096 with a
# model width of 2048 (16 heads of 128 or 32 of 64), and a grouped-query
# shape (32 query heads over 8 key/value heads of 128) at 8192.
ATTN_WORKLOADS = {
    w.name: w for w in [
        AttnWorkload("attn_d128_n4096", 20, 4, 16, 16, 4096, 128, False),
        AttnWorkload("attn_d128_n4096_causal", 20, 4, 16, 16, 4096, 128, True),
        AttnWorkload("attn_d64_n4096", 21, 4, 32, 32, 4096, 64, False),
        AttnWorkload("attn_gqa_d128_n8192_causal", 22, 1, 32, 8, 8192, 128, True),
    ]
}


def make_attn_inputs(w: AttnWorkload):
    """dict(q, k, v) as packed bf16 CPU tensors; workload index c seeds q, k, v
    with 1000c + 1, + 2, + 3."""
    out = {}
    for i, (name, H) in enumerate((("q", w.Hq), ("k", w.Hkv), ("v", w.Hkv))):
        g = _gen(1000 * w.index + 1 + i)
        out[name] = torch.randn(w.B, H, w.N, w.D, generator=g, dtype=torch.float32).to(
            torch.bfloat16)
    return out


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def bf16_matrix(rows: int, cols: int, dist: str, seed: int) -> torch.Tensor:
    """A rows x cols bfloat16 CPU tensor; each entry is rounded to bf16 once."""
    g = _gen(seed)
    if dist == "uniform":
        x = torch.rand(rows, cols, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "normal":
        x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    elif dist == "normal002":
        x = torch.randn(rows, cols, generator=g, dtype=torch.float32) * 0.02
    elif dist == "int4":
        x = torch.randint(-4, 5, (rows, cols), generator=g).to(torch.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    return x.to(torch.bfloat16)


def fp8_matrix(rows: int, cols: int, seed: int, integer: bool = False):
    """(e4m3 bytes as a uint8 CPU tensor, fp32 scale) for one operand.

    Normal(0, 1) draws are divided by s = amax / 448, clamped to +-448 (the
    float8 cast does not saturate) and rounded to e4m3 once, so that
    x ~= s * q.  The integer variant draws {-4..4}, which e4m3 holds exactly,
    with scale 1.
    """
    g = _gen(seed)
    if integer:
        x = torch.randint(-4, 5, (rows, cols), generator=g).to(torch.float32)
        q = x.to(torch.float8_e4m3fn)
        return q.view(torch.uint8), 1.0
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    amax = float(x.abs().max())
    s = torch.tensor(amax / E4M3_MAX, dtype=torch.float32)
    q = torch.clamp(x / s, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), float(s)


def mxfp8_matrix(rows: int, cols: int, seed: int, integer: bool = False):
    """(e4m3 bytes (rows, cols), E8M0 scale bytes (rows, ceil(cols/32))) as uint8 CPU tensors.

    Normal(0, 1) draws, quantised per block of 32 consecutive values of a row:
    shared exponent e = floor(log2 amax) - 8 (8 = the exponent of e4m3's
    largest normal, 448 = 1.75 * 2^8), scale byte e + 127 clamped to [0, 254],
    elements x * 2^-e clamped to +-448 and rounded to e4m3 once.  An all-zero
    block gets scale byte 127.  The integer variant draws elements in {-4..4}
    and scale bytes in {126, 127, 128}, so that every sum of products is a
    multiple of 1/4 below 2^21 for K up to 8192: exact in fp32.
    """
    g = _gen(seed)
    nb = (cols + 31) // 32
    if integer:
        x = torch.randint(-4, 5, (rows, cols), generator=g).to(torch.float32)
        sc = torch.randint(126, 129, (rows, nb), generator=g).to(torch.uint8)
        return x.to(torch.float8_e4m3fn).view(torch.uint8), sc
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    xp = torch.zeros(rows, nb * 32, dtype=torch.float32)
    xp[:, :cols] = x
    blocks = xp.view(rows, nb, 32)
    amax = blocks.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 8, torch.zeros_like(amax))
    e = torch.clamp(e, -127, 127)
    q = torch.clamp(blocks * torch.exp2(-e).unsqueeze(2), -E4M3_MAX, E4M3_MAX)
    q = q.view(rows, nb * 32)[:, :cols].contiguous().to(torch.float8_e4m3fn)
    sc = (e + 127).to(torch.uint8)
    return q.view(torch.uint8), sc


def make_inputs(w: Workload, integer: bool = False):
    """Return dict(A=..., B=..., scale_a=..., scale_b=...) as CPU tensors.

    bf16 operands are torch.bfloat16; fp8 operands are uint8 e4m3 bytes.
    """
    sa_seed, sb_seed = w.seeds(integer)
    if w.dtype == "bf16":
        dist = "int4" if integer else w.dist
        A = bf16_matrix(w.M, w.K, dist, sa_seed)
        B = bf16_matrix(w.N, w.K, dist, sb_seed)
        return {"A": A, "B": B, "scale_a": 1.0, "scale_b": 1.0}
    if w.dtype == "mxfp8":
        A, SA = mxfp8_matrix(w.M, w.K, sa_seed, integer)
        B, SB = mxfp8_matrix(w.N, w.K, sb_seed, integer)
        return {"A": A, "B": B, "SA": SA, "SB": SB, "scale_a": 1.0, "scale_b": 1.0}
    A, sa = fp8_matrix(w.M, w.K, sa_seed, integer)
    B, sb = fp8_matrix(w.N, w.K, sb_seed, integer)
    return {"A": A, "B": B, "scale_a": sa, "scale_b": sb}


def stored(w: Workload, x: dict):
    """(A, B) as the workload's layout stores them: the logical M x K and N x K
    matrices, or their transposes (K x M, K x N) for a layout of 1."""
    A = x["A"].t().contiguous() if w.layout_a else x["A"]
    B = x["B"].t().contiguous() if w.layout_b else x["B"]
    return A, B


def bits(t: torch.Tensor):
    """numpy view of a tensor's raw bit patterns (uint16 for bf16, uint8 for e4m3)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.contiguous().view(torch.uint8).numpy()
    raise TypeError("unsupported dtype %s" % t.dtype)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(bits(t).tobytes()).hexdigest()
