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
                      max |x| = 448, rounded to OCP e4m3, with fp32 scales.

Seeds: workload index c gives A seed 1000c+1 and B seed 1000c+2; the integer
variant adds 10.
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
    dtype: str   # "bf16" or "fp8"
    dist: str    # "uniform", "normal", "normal002", "int4", "fp8_normal"

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 1

    @property
    def algorithmic_bytes(self) -> int:
        """Read each input once, write C (bf16) once."""
        return (self.M + self.N) * self.K * self.in_bytes + 2 * self.M * self.N

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
    ]
}


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
    A, sa = fp8_matrix(w.M, w.K, sa_seed, integer)
    B, sb = fp8_matrix(w.N, w.K, sb_seed, integer)
    return {"A": A, "B": B, "scale_a": sa, "scale_b": sb}


def bits(t: torch.Tensor):
    """numpy view of a tensor's raw bit patterns (uint16 for bf16, uint8 for e4m3)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view("uint16")
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.contiguous().view(torch.uint8).numpy()
    raise TypeError("unsupported dtype %s" % t.dtype)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(bits(t).tobytes()).hexdigest()
