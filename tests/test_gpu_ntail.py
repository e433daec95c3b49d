"""GPU parity for N that is not a multiple of 64 (narrowed last column tile).

The pages' kernels require N to be a multiple of 64 ("Aligned shared rows
for pipelined NAX on CUDA", section "Contract and correctness"); this
library serves any positive N with B stored [N,K] and multiples of 8 with B
stored [K,N].  The operation and the acceptance are unchanged: partials and
C against the binary64 oracle within the pages' tolerances, NaN-poisoned
outputs (every element inside N written), guards after every buffer
untouched (nothing written past the ends).  A write to a column at or past N
would land in the next row and fail the element comparison.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

PARTIAL_TOL = 1e-4
FINAL_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}
GUARD_BITS = np.float32(inputs.GUARD_VALUE).view(np.uint32)

# (M, N, K, kps, splits): N below one tile, odd N, N % 4 != 0 (rows not
# 16-byte aligned), tails of every size class, several tiles plus a tail.
NK_SHAPES = [
    (32, 1, 64, 32, 2),
    (32, 3, 256, 128, 2),
    (64, 36, 512, 256, 2),
    (96, 100, 2048, 512, 4),
    (32, 130, 2080, 544, 4),
    (64, 200, 1056, 1024, 2),
    (160, 520, 608, 96, 7),
    (256, 1000, 2048, 1024, 2),
    (32, 1030, 4096, 1024, 4),
]
KN_SHAPES = [(M, N, K, kps, S) for M, N, K, kps, S in
             [(32, 8, 64, 32, 2), (64, 40, 512, 256, 2), (96, 104, 2048, 512, 4),
              (32, 136, 2080, 544, 4), (160, 520, 608, 96, 7), (256, 1000, 2048, 1024, 2)]]


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _vals(t):
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


def _run(sdg, a, b, kps, S, layout, plan=None):
    dev = torch.device("cuda:0")
    M, N = a.shape[0], b.shape[0]
    pbuf = inputs.guarded_buffer(S * M * N, "nan").to(dev)
    cbuf = inputs.guarded_buffer(M * N, "nan").to(dev)
    P, C = pbuf[: S * M * N].view(S, M, N), cbuf[: M * N].view(M, N)
    bd = b.to(dev) if layout == "nk" else b.T.contiguous().to(dev)
    if plan:
        sdg.gemm_planned(plan, a.to(dev), bd, P, kps, S, C=C, layout=layout)
    elif layout == "nk":
        sdg.gemm_bt_reduce(a.to(dev), bd, P, C, kps, S)
    else:
        sdg.gemm_bn_reduce(a.to(dev), bd, P, C, kps, S)
    torch.cuda.synchronize()
    p, c = pbuf.cpu().numpy(), cbuf.cpu().numpy()
    assert np.all(p[S * M * N:].view(np.uint32) == GUARD_BITS), "a partials guard changed"
    assert np.all(c[M * N:].view(np.uint32) == GUARD_BITS), "a guard after C changed"
    return p[: S * M * N].reshape(S, M, N), c[: M * N].reshape(M, N)


def _check(sdg, M, N, K, kps, S, dtype, layout, seed, plan=None):
    a, b = inputs.make_operands(M, N, K, dtype, seed=seed, zero_first_row=True, scale_last_row=True)
    P, C = _run(sdg, a, b, kps, S, layout, plan)
    a64, b64 = _vals(a), _vals(b)
    RP, DP, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    ep, _ = oracle.normalized_error(P, RP, DP)
    ec, _ = oracle.normalized_error(C, RC, DC)
    print(f"  partial err {ep:.3e}, final err {ec:.3e}", flush=True)
    assert ep <= PARTIAL_TOL and ec <= FINAL_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", NK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nk_tails(sdg, shape, dtype):
    M, N, K, kps, S = shape
    print(f"case nk tail {dtype} M{M} N{N} K{K} kps{kps} S{S}: "
          f"{sdg.describe(M, N, K, kps, S, inputs.DTYPES[dtype])}", flush=True)
    _check(sdg, M, N, K, kps, S, dtype, "nk", seed=N + K + S)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", KN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_kn_tails(sdg, shape, dtype):
    M, N, K, kps, S = shape
    print(f"case kn tail {dtype} M{M} N{N} K{K} kps{kps} S{S}: "
          f"{sdg.describe_bn(M, N, K, kps, S, inputs.DTYPES[dtype])}", flush=True)
    _check(sdg, M, N, K, kps, S, dtype, "kn", seed=N * 3 + K + S)


@pytest.mark.parametrize("layout", ["nk", "kn"])
@pytest.mark.parametrize("plan", ["tiled,256,256,2,2", "tiled,256,128,2,2"])
def test_tiled_tails_forced(sdg, layout, plan):
    """The large-tile kernels with a narrowed last tile (40 columns)."""
    M, N, K, kps, S = 256, 296, 1248, 608, 3
    desc = sdg.describe_planned(plan, M, N, K, kps, S, torch.bfloat16, layout=layout)
    print(f"case {layout} {plan} M{M} N{N}: {desc}", flush=True)
    assert desc.startswith("tiled bm256 bn" + plan.split(",")[2])
    _check(sdg, M, N, K, kps, S, "bf16", layout, seed=17, plan=plan)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tails_exact_bitwise(sdg, dtype):
    for layout, (M, N, K, kps, S) in (("nk", (96, 100, 480, 160, 3)), ("nk", (32, 3, 256, 128, 2)),
                                      ("kn", (96, 104, 480, 160, 3))):
        a, b = inputs.exact_operands(M, N, K, dtype, seed=N)
        P, C = _run(sdg, a, b, kps, S, layout)
        a64, b64 = _vals(a), _vals(b)
        RP, _, _ = oracle.splitk_partials(a64, b64, kps, S)
        RC, _, _ = oracle.gemm_bt(a64, b64)
        np.testing.assert_array_equal(P.astype(np.float64), RP)
        np.testing.assert_array_equal(C.astype(np.float64), RC)


def test_large_tail_sampled(sdg):
    """2048 x 4000 x 1024 in 4 splits: 256x128 tiles, the last one 32 wide."""
    M, N, K, kps, S = 2048, 4000, 1024, 256, 4
    desc = sdg.describe(M, N, K, kps, S, torch.bfloat16)
    print(f"case large tail {desc}", flush=True)
    a, b = inputs.make_operands(M, N, K, "bf16", seed=23)
    P, C = _run(sdg, a, b, kps, S, "nk")
    assert not np.isnan(P).any() and not np.isnan(C).any()
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.integers(0, M, 2044), [0, M - 1, 0, M - 1]])
    cols = np.concatenate([rng.integers(3968, N, 1024), rng.integers(0, N, 1020), [0, N - 1, N - 1, 0]])
    SP, SDP, SC, SDC = oracle.sampled(_vals(a), _vals(b), kps, S, rows, cols)
    assert oracle.normalized_error(P[:, rows, cols].T, SP, SDP)[0] <= PARTIAL_TOL
    assert oracle.normalized_error(C[rows, cols], SC, SDC)[0] <= FINAL_TOL["bf16"]


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_auto_with_tail(sdg, out):
    dev = torch.device("cuda:0")
    M, N, K = 64, 1000, 4096
    a, b = inputs.make_operands(M, N, K, "bf16", seed=29)
    kps, S, need = sdg.choose_splits(M, N, K, torch.bfloat16, inputs.DTYPES[out])
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    ws = torch.empty(max(need, 1), device=dev)
    sdg.gemm_bt_auto(a.to(dev), b.to(dev), cbuf[: M * N].view(M, N), workspace=ws[:need] if need else None)
    torch.cuda.synchronize()
    bits = inputs.stored_bits(cbuf.cpu())
    guard = inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[out]))[0]
    assert np.all(bits[M * N:] == guard)
    RC, DC, _ = oracle.gemm_bt(_vals(a), _vals(b))
    err, _ = oracle.normalized_error(oracle.decode(bits[: M * N], out).reshape(M, N), RC, DC)
    assert err <= FINAL_TOL["bf16"]


@pytest.mark.parametrize("N", [1, 3, 36, 1000])
def test_reduce_tail_planes(sdg, N):
    dev = torch.device("cuda:0")
    M, S = 32, 5
    gen = torch.Generator().manual_seed(N)
    slabs = torch.randint(-999, 999, (S, M, N), generator=gen).float().div_(16)
    for out in ("f32", "f16"):
        cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
        sdg.reduce(slabs.to(dev), cbuf[: M * N].view(M, N), S)
        torch.cuda.synchronize()
        bits = inputs.stored_bits(cbuf.cpu())
        ref, _, _ = oracle.slab_sum(slabs.numpy())
        np.testing.assert_array_equal(bits[: M * N], oracle.encode(ref, out).ravel())
