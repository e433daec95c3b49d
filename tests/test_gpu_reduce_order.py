"""GPU: the slab sum in a GEMM's tile order (splitk_reduce_for_gemm, also
run by every fused call) against the flat slab sum and the binary64
reference.

The accumulation pass is the separate elementwise sum of the slabs ("Aligned
shared rows for pipelined NAX on CUDA", section "Contract and correctness").
The tile-ordered pass only changes which workgroup visits which part of the
plane, so its output must equal the flat pass bit for bit (both add the
slabs in ascending s in F32), for every output type, with NaN-poisoned
outputs fully overwritten and the 64 guards intact.  Geometries cover both
small tile shapes, a forced 64x64 tile, tile counts that are and are not
multiples of the 8 XCDs, column tails, and the cases that fall back to the
flat order (N % 4 != 0, more than eight slabs, large-tile GEMMs past one
round of workgroups or 32 MiB of slabs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

GUARD_BITS = np.float32(inputs.GUARD_VALUE).view(np.uint32)
GUARD16 = {d: int(inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[d]))[0])
           for d in ("f16", "bf16")}

# (M, N, K, k_per_split, splits, input dtype, forced plan or None, tile order expected)
GEOMETRIES = [
    (256, 1024, 2048, 1024, 2, "bf16", None, True),    # 32x64 tiles, 128 of them
    (96, 512, 2048, 512, 4, "bf16", None, True),       # 32x32 tiles, 48
    (32, 512, 2080, 544, 4, "f16", None, True),        # 32x32, 16 tiles, short last split
    (96, 320, 1024, 256, 4, "bf16", None, True),       # 30 tiles: not a multiple of 8
    (96, 200, 1024, 512, 2, "bf16", None, True),       # column tail (N % 4 == 0)
    (64, 100, 512, 256, 2, "f32", None, True),         # F32 plan, column tail
    (64, 256, 2048, 256, 8, "bf16", None, True),       # eight slabs (largest tile-order count)
    (128, 256, 1024, 512, 2, "bf16", "wavek,64,64,4,2", True),   # forced 64x64 tiles
    (64, 768, 12288, 1536, 8, "bf16", None, False),    # long K: split-major order, flat pass
    (64, 130, 512, 256, 2, "bf16", None, False),       # N % 4 != 0: flat order
    (32, 64, 2048, 128, 16, "bf16", None, False),      # sixteen slabs: flat order
    (2048, 2048, 1024, 512, 2, "bf16", None, True),    # 256x128 tiles, one round, 32 MiB of slabs
    (2048, 4096, 1024, 512, 2, "bf16", None, False),   # large tiles, 64 MiB of slabs: flat order
]


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _slabs(M, N, S, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(S, M, N, generator=gen) * 3


def _run(sdg, fn_name, slabs, M, N, geo, out):
    K, kps, S, dt = geo[2], geo[3], geo[4], geo[5]
    dev = torch.device("cuda:0")
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    C = cbuf[: M * N].view(M, N)
    P = slabs.to(dev)
    if fn_name == "flat":
        sdg.reduce(P, C, S)
    else:
        sdg.reduce_for_gemm(P, C, K, kps, S, inputs.DTYPES[dt])
    torch.cuda.synchronize()
    return inputs.stored_bits(cbuf.cpu())


def _run_planned(sdg, plan, M, N, geo, out):
    """The fused call with a named GEMM configuration; returns C's stored
    bits (guards included) and the slabs the GEMM wrote."""
    K, kps, S, dt = geo[2], geo[3], geo[4], geo[5]
    dev = torch.device("cuda:0")
    a, b = inputs.make_operands(M, N, K, dt, seed=M + N + S)
    P = torch.empty(S, M, N, device=dev)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    sdg.gemm_planned(plan, a.to(dev), b.to(dev), P, kps, S, C=cbuf[: M * N].view(M, N))
    torch.cuda.synchronize()
    return inputs.stored_bits(cbuf.cpu()), P.cpu()


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("geo", GEOMETRIES, ids=lambda g: "x".join(map(str, g[:5])) + f"-{g[5]}"
                         + ("-forced" if g[6] else "") + ("-tiles" if g[7] else "-flat"))
def test_tile_order_equals_flat_order(sdg, geo, out):
    M, N, K, kps, S, dt, plan, tile_order = geo
    if plan:
        text = sdg.describe_planned(plan, M, N, K, kps, S, inputs.DTYPES[dt])
    else:
        text = sdg.describe(M, N, K, kps, S, inputs.DTYPES[dt])
    print(f"reduce order: {geo} out={out} plan={text}", flush=True)
    assert ("splitfast" in text) == tile_order, text
    if plan:
        # A named configuration: its fused call (the GEMM, then the pass in
        # that GEMM's tile order) against the flat pass over its own slabs.
        got, slabs = _run_planned(sdg, plan, M, N, geo, out)
    else:
        slabs = _slabs(M, N, S, seed=M + N + S)
        got = _run(sdg, "tile", slabs, M, N, geo, out)
    flat = _run(sdg, "flat", slabs, M, N, geo, out)
    np.testing.assert_array_equal(got, flat)
    guard = GUARD_BITS if out == "f32" else GUARD16[out]
    assert np.all(got[M * N:] == guard)
    if out == "f32":
        vals = got[: M * N].view(np.float32)
        assert not np.isnan(vals).any()
        ref, D, _ = oracle.slab_sum(slabs.numpy())
        err, _ = oracle.normalized_error(vals, ref, D)
        assert err <= max(S - 1, 0) * 2.0**-24 * 1.0001


def test_fused_chain_runs_the_tile_order(sdg):
    """The fused call's C equals the separate GEMM followed by either pass,
    bit for bit, on the headline workload."""
    w = inputs.WORKLOADS["bf16_m256_n1024_k2048_s2"]
    a, b = inputs.workload_operands(w)
    dev = torch.device("cuda:0")
    A, B = a.to(dev), b.to(dev)
    P = torch.empty(w.splits, w.M, w.N, device=dev)
    C1, C2, C3 = (torch.full((w.M, w.N), float("nan"), device=dev) for _ in range(3))
    sdg.gemm_bt_reduce(A, B, P, C1, w.kps, w.splits)
    sdg.reduce(P, C2, w.splits)
    sdg.reduce_for_gemm(P, C3, w.K, w.kps, w.splits, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2) and torch.equal(C1, C3)


def test_reduce_for_gemm_statuses(sdg):
    """Bad geometry, dtype or pointers are rejected before anything runs."""
    dev = torch.device("cuda:0")
    pool = torch.zeros(1 << 20, dtype=torch.float32, device=dev)
    P, C = pool.data_ptr(), pool.data_ptr() + (1 << 21)
    call = lambda *a: sdg.raw_call("splitk_reduce_for_gemm", *a)  # noqa: E731
    bf = inputs.DTYPE_CODES["bf16"]
    assert call(None, C, 64, 128, 256, 128, 2, bf, 0, None) == 1
    assert call(P, None, 64, 128, 256, 128, 2, bf, 0, None) == 1
    assert call(P, C, 64, 128, 256, 128, 2, 7, 0, None) == 2
    assert call(P, C, 64, 128, 256, 128, 2, bf, 5, None) == 2
    assert call(P, C, 48, 128, 256, 128, 2, bf, 0, None) == 3
    assert call(P, C, 64, 128, 256, 128, 3, bf, 0, None) == 4    # splits do not match K
    assert call(P, C, 64, 128, 256, 96, 2, bf, 0, None) == 4     # splits do not cover K
    assert call(P + 4, C, 64, 128, 256, 128, 2, bf, 0, None) == 6
    assert call(P, P + 1024, 64, 128, 256, 128, 2, bf, 0, None) == 5
    torch.cuda.synchronize()
    assert torch.count_nonzero(pool).item() == 0
