"""Seeded synthetic inputs for split-K GEMM.

This module only draws and lays out input data: it holds none of the GEMM or
reduction arithmetic, and both the HIP path's callers and the F64 reference's
callers take their operands from here.

Shapes and value recipes follow the workloads the pages measure
("Aligned shared rows for pipelined NAX on CUDA", sections "Contract and
correctness" and "Measurement protocol"; "Wider consecutive-weight NAX GEMM",
sections "Launch contract and correctness" and "Performance method"):
row-major A[M,K] and B[N,K] in F32, F16 or BF16, finite and inside the F16
range; test inputs have a zero first A row and a last A row at four times the
ordinary scale; partial buffers start poisoned at 7 with 64 trailing guard
elements at 11.

Recipe: draw F32 values with a seeded ``torch.Generator`` (A first, then B),
then round to the element type with round-to-nearest-even (``Tensor.to``).
The x4 row scale is a power of two and so commutes with that rounding; it is
applied after it.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
ELEMENT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

GUARD_COUNT = 64
GUARD_VALUE = 11.0
POISON_VALUE = 7.0
NAN_POISON_BITS = 0x7FC00000  # quiet NaN


@dataclasses.dataclass(frozen=True)
class Workload:
    """One split-K GEMM problem: shapes, split geometry and value recipe."""

    name: str
    dtype: str
    M: int
    N: int
    K: int
    kps: int
    splits: int
    dist: str = "uniform"  # "uniform" = U[-1,1]; "normal" = N(0, 0.5) clipped to +-4
    seed: int = 0
    zero_first_row: bool = False
    scale_last_row: bool = False

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def split_lengths(self) -> list[int]:
        return [min(self.K, (s + 1) * self.kps) - s * self.kps for s in range(self.splits)]


# The five measured and tested configurations, named by what they are: the
# smallest case, the two shapes the first page's headline names, a skinny
# F16 case whose last split is short, and a large case.
CONFIGS = (
    Workload("f32_m32_n64_k64_s2", "f32", 32, 64, 64, 32, 2, seed=1234,
             zero_first_row=True, scale_last_row=True),
    Workload("bf16_m96_n512_k2048_s4", "bf16", 96, 512, 2048, 512, 4, seed=1235),
    Workload("bf16_m256_n1024_k2048_s2", "bf16", 256, 1024, 2048, 1024, 2, seed=1236,
             zero_first_row=True, scale_last_row=True),
    Workload("f16_m32_n512_k2080_s4", "f16", 32, 512, 2080, 544, 4, seed=1237),
    Workload("bf16_m2048_n4096_k4096_s8", "bf16", 2048, 4096, 4096, 512, 8, dist="normal",
             seed=1238),
)

# The other (dtype, shape, split) rows the pages time, with seeded uniform
# [-1,1] inputs: "Aligned shared rows for pipelined NAX on CUDA", table of
# the section "Measurement protocol" (256x512x2048 at 2 splits in BF16 and
# F16, 96x512x2048 at 4 splits in F16 and F32, 96x512x512 at 4 splits,
# 32x64x32 at 1 split), and "Wider consecutive-weight NAX GEMM", table of
# the section "Performance method" (256x512x2048 at 4 splits in BF16, F16
# and F32, 128x512x2048 at 8 splits, 96x512x2048 at 8 splits) and its
# skinny 32-row case at 4 splits.
PAGE_SHAPES = (
    Workload("bf16_m256_n512_k2048_s2", "bf16", 256, 512, 2048, 1024, 2, seed=1239),
    Workload("f16_m256_n512_k2048_s2", "f16", 256, 512, 2048, 1024, 2, seed=1240),
    Workload("f16_m96_n512_k2048_s4", "f16", 96, 512, 2048, 512, 4, seed=1241),
    Workload("f32_m96_n512_k2048_s4", "f32", 96, 512, 2048, 512, 4, seed=1242),
    Workload("bf16_m96_n512_k512_s4", "bf16", 96, 512, 512, 128, 4, seed=1243),
    Workload("bf16_m32_n64_k32_s1", "bf16", 32, 64, 32, 32, 1, seed=1244),
    Workload("bf16_m256_n512_k2048_s4", "bf16", 256, 512, 2048, 512, 4, seed=1245),
    Workload("f16_m256_n512_k2048_s4", "f16", 256, 512, 2048, 512, 4, seed=1246),
    Workload("f32_m256_n512_k2048_s4", "f32", 256, 512, 2048, 512, 4, seed=1247),
    Workload("bf16_m128_n512_k2048_s8", "bf16", 128, 512, 2048, 256, 8, seed=1248),
    Workload("bf16_m96_n512_k2048_s8", "bf16", 96, 512, 2048, 256, 8, seed=1249),
    Workload("bf16_m32_n512_k2048_s4", "bf16", 32, 512, 2048, 512, 4, seed=1250),
)

WORKLOADS = {w.name: w for w in CONFIGS + PAGE_SHAPES}

# Shapes whose N the column tile does not divide (the N-tail tiles), for the
# measurements of the calls beyond the fixed chain: the headline and large
# shapes with N cut below a multiple of 64 and of 256, and skinny F16 and F32
# cases.  Same recipe as above.
NTAIL_SHAPES = (
    Workload("bf16_m256_n1000_k2048_s2", "bf16", 256, 1000, 2048, 1024, 2, seed=1260),
    Workload("f16_m32_n520_k2080_s4", "f16", 32, 520, 2080, 544, 4, seed=1261),
    Workload("f32_m96_n504_k2048_s4", "f32", 96, 504, 2048, 512, 4, seed=1262),
    Workload("bf16_m2048_n4000_k4096_s8", "bf16", 2048, 4000, 4096, 512, 8, dist="normal", seed=1263),
)

HEADLINE = "bf16_m256_n1024_k2048_s2"


def _draw(gen: torch.Generator, shape, dist: str) -> torch.Tensor:
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32).mul_(2.0).sub_(1.0)
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32).mul_(0.5).clamp_(-4.0, 4.0)
    raise ValueError(f"unknown distribution {dist!r}")


def make_operands(M: int, N: int, K: int, dtype: str, seed: int, dist: str = "uniform",
                  zero_first_row: bool = False, scale_last_row: bool = False):
    """CPU tensors A[M,K] and B[N,K] of element type `dtype`."""
    gen = torch.Generator().manual_seed(seed)
    a = _draw(gen, (M, K), dist).to(DTYPES[dtype])
    b = _draw(gen, (N, K), dist).to(DTYPES[dtype])
    if zero_first_row:
        a[0].zero_()
    if scale_last_row and M > 1:
        a[M - 1].mul_(4)
    return a.contiguous(), b.contiguous()


def workload_operands(w: Workload):
    return make_operands(w.M, w.N, w.K, w.dtype, w.seed, w.dist, w.zero_first_row, w.scale_last_row)


def exact_operands(M: int, N: int, K: int, dtype: str, seed: int):
    """Operands whose entries are j/8 with integer |j| <= 8.

    Every such value is exact in F32, F16 and BF16, every product is a
    multiple of 1/64, and for K <= 2**17 every partial sum stays an integer
    multiple of 1/64 below 2**18 in magnitude, so F32 accumulation in any
    order is exact.
    """
    gen = torch.Generator().manual_seed(seed)
    a = torch.randint(-8, 9, (M, K), generator=gen).to(torch.float32).div_(8)
    b = torch.randint(-8, 9, (N, K), generator=gen).to(torch.float32).div_(8)
    return a.to(DTYPES[dtype]).contiguous(), b.to(DTYPES[dtype]).contiguous()


def product_factors(M: int, N: int, K: int, seed: int, a_max: int = 3, b_max: int = 5):
    """Seeded integer factors (a[M], b[N], u[K], v[K]) of the operands
    A[i,k] = a[i]*u[k] and B[j,k] = b[j]*v[k] (``product_operands``).

    a[i] is drawn from +-1..a_max, b[j] from +-1..b_max, u[k] and v[k] from
    {-1, 0, 1}, all uniformly; CPU int64 tensors.  Every operand entry is then
    an integer of magnitude at most a_max or b_max, exact in F32, F16 and BF16.
    """
    gen = torch.Generator().manual_seed(seed)

    def signed(n, top):
        mag = torch.randint(1, top + 1, (n,), generator=gen)
        return mag * (torch.randint(0, 2, (n,), generator=gen) * 2 - 1)

    a = signed(M, a_max)
    b = signed(N, b_max)
    u = torch.randint(-1, 2, (K,), generator=gen)
    v = torch.randint(-1, 2, (K,), generator=gen)
    return a, b, u, v


def product_operands(factors, dtype: str, device, b_layout: str = "nk"):
    """A[M,K] = a (x) u and B = b (x) v from ``product_factors``, built directly
    in element type `dtype` on `device` (each entry is one exact product of two
    small integers).  B is [N,K] for b_layout "nk" and [K,N] for "kn"."""
    a, b, u, v = factors
    t = DTYPES[dtype]
    a_, b_, u_, v_ = (x.to(device=device, dtype=t) for x in (a, b, u, v))
    A = torch.outer(a_, u_).contiguous()
    B = torch.outer(b_, v_) if b_layout == "nk" else torch.outer(v_, b_)
    return A, B.contiguous()


def guarded_buffer(n: int, poison: str = "seven", dtype: str = "f32") -> torch.Tensor:
    """CPU buffer of n poisoned elements of `dtype` plus GUARD_COUNT trailing guards."""
    buf = torch.empty(n + GUARD_COUNT, dtype=DTYPES[dtype])
    if poison == "seven":
        buf[:n] = POISON_VALUE
    elif poison == "nan":
        if dtype == "f32":
            buf[:n].view(torch.int32).fill_(NAN_POISON_BITS)
        else:
            buf[:n] = float("nan")
    else:
        raise ValueError(poison)
    buf[n:] = GUARD_VALUE
    return buf


def stored_bits(t: torch.Tensor) -> np.ndarray:
    """The stored bit patterns of a CPU tensor: uint16 for F16/BF16, uint32 for F32."""
    t = t.contiguous().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def dtype_name(t: torch.Tensor) -> str:
    for k, v in DTYPES.items():
        if v == t.dtype:
            return k
    raise TypeError(t.dtype)
