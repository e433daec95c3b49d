"""Seeded random geometries against the binary64 oracle.

Each case draws M (multiple of 32), N (any, or a multiple of 8 for B stored
[K,N]), K (multiple of 32), a split count and the matching k_per_split, an
input type, a B layout and an output type, then checks partials and C with
the tolerances of "Aligned shared rows for pipelined NAX on CUDA", section
"Contract and correctness" (final C per input type when F32, per output type
when F16/BF16), NaN-poisoned outputs and trailing guards.  The cases are
fixed by the seed, so a failure names a reproducible geometry.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

FINAL_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}
GUARD_BITS = np.float32(inputs.GUARD_VALUE).view(np.uint32)


def _cases(n=60, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        layout = "kn" if rng.random() < 0.35 else "nk"
        M = 32 * int(rng.integers(1, 11))
        N = int(rng.integers(1, 90)) * 8 if layout == "kn" else int(rng.integers(1, 700))
        K = 32 * int(rng.integers(1, 81))
        S = int(rng.integers(1, min(8, K // 32) + 1))
        kps = 32 * -(-(K // 32) // S)
        while (S - 1) * kps >= K:  # the split count that geometry actually needs
            S -= 1
        dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
        out_t = ["f32", "f32", "f16", "bf16"][int(rng.integers(0, 4))]
        out.append((i, layout, M, N, K, kps, S, dtype, out_t))
    return out


def _large_cases(n=20, seed=20261203):
    """Geometries for the large-tile kernels: M a multiple of 256 up to 2048,
    N from ~1900 to ~4200 (mostly not a multiple of 256), K up to 2080, 3-8
    splits,
    so that the draws reach the one-tile 256x128 and 256x256 kernels, their
    persistent form (more 256x256 tiles than CUs), narrowed last column
    tiles and the split-fastest order of one-round grids, in both layouts."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        layout = "kn" if rng.random() < 0.4 else "nk"
        M = 256 * int(rng.integers(2, 9))
        N = 8 * int(rng.integers(250, 525)) if layout == "kn" else int(rng.integers(1900, 4200))
        S = int(rng.integers(3, 9))
        K = 32 * int(rng.integers(2 * S, 66))
        kps = 32 * -(-(K // 32) // S)
        while (S - 1) * kps >= K:
            S -= 1
        dtype = ["f32", "f16", "bf16", "bf16"][int(rng.integers(0, 4))]
        out_t = ["f32", "f32", "f16", "bf16"][int(rng.integers(0, 4))]
        out.append((100 + i, layout, M, N, K, kps, S, dtype, out_t))
    return out


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _vals(t):
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


@pytest.mark.parametrize("case", _cases() + _large_cases(), ids=lambda c: "r{}-{}-{}x{}x{}-s{}-{}-{}".format(
    c[0], c[1], c[2], c[3], c[4], c[6], c[7], c[8]))
def test_random_geometry(sdg, case):
    i, layout, M, N, K, kps, S, dtype, out_t = case
    assert (S - 1) * kps < K <= S * kps
    describe = sdg.describe if layout == "nk" else sdg.describe_bn
    print(f"case {case}: {describe(M, N, K, kps, S, inputs.DTYPES[dtype])}", flush=True)
    dev = torch.device("cuda:0")
    a, b = inputs.make_operands(M, N, K, dtype, seed=1000 + i, zero_first_row=bool(i % 2),
                                scale_last_row=bool(i % 3 == 0))
    pbuf = inputs.guarded_buffer(S * M * N, "nan").to(dev)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out_t).to(dev)
    P, C = pbuf[: S * M * N].view(S, M, N), cbuf[: M * N].view(M, N)
    if layout == "nk":
        sdg.gemm_bt_reduce(a.to(dev), b.to(dev), P, C, kps, S)
    else:
        sdg.gemm_bn_reduce(a.to(dev), b.T.contiguous().to(dev), P, C, kps, S)
    torch.cuda.synchronize()
    p = pbuf.cpu().numpy()
    cbits = inputs.stored_bits(cbuf.cpu())
    assert np.all(p[S * M * N:].view(np.uint32) == GUARD_BITS)
    guard_c = inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[out_t]))[0]
    assert np.all(cbits[M * N:] == guard_c)
    a64, b64 = _vals(a), _vals(b)
    RP, DP, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    ep, _ = oracle.normalized_error(p[: S * M * N], RP, DP)
    ec, _ = oracle.normalized_error(oracle.decode(cbits[: M * N], out_t), RC, DC)
    tol = FINAL_TOL[dtype] if out_t == "f32" else FINAL_TOL[out_t]
    print(f"  partial err {ep:.3e}, final err {ec:.3e} (tolerance {tol})", flush=True)
    assert ep <= 1e-4 and ec <= tol
