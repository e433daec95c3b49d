"""GPU parity of the split-K GEMM with B stored [K,N] (splitk_gemm_bn).

The operation is the one of "Aligned shared rows for pipelined NAX on CUDA",
section "Contract and correctness": partials[s,i,j] is the sum over split
s's k range of A[i,k]*B[k,j], here with B's rows holding n instead of k
("Wider consecutive-weight NAX GEMM", section "Performance method", prepares
weights in both orders).  The reference is the binary64 oracle applied to the
same values read as [N,K] (the transpose of the stored [K,N] array), with the
pages' tolerances, NaN-poisoned outputs and guards after every buffer.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from conftest import LARGEST, largest_reference
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

PARTIAL_TOL = 1e-4
FINAL_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}
GUARD_BITS = np.float32(inputs.GUARD_VALUE).view(np.uint32)

SHAPES = [
    (32, 64, 32, 32, 1),
    (64, 192, 256, 128, 2),
    (32, 512, 2080, 544, 4),     # 16-bit splits ending in half chunks
    (96, 320, 480, 160, 3),
    (32, 64, 8192, 2048, 4),
    (96, 512, 2048, 512, 4),
    (256, 1024, 2048, 1024, 2),
    (64, 128, 1056, 1024, 2),    # final split of 32
    (160, 192, 608, 96, 7),
    (512, 1024, 1024, 256, 4),   # large tiles
    (256, 768, 1120, 576, 2),    # large tiles, 256-wide column tiles not possible
]


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _vals(t):
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


def run_bn(sdg, a, b_nk, kps, S, out="f32", poison="nan"):
    """Runs gemm_bn_reduce with B passed as the [K,N] array b_nk^T.
    Returns (partials, C bits) and checks the guards."""
    dev = torch.device("cuda:0")
    M, K = a.shape
    N = b_nk.shape[0]
    b_kn = b_nk.T.contiguous()
    pbuf = inputs.guarded_buffer(S * M * N, poison).to(dev)
    cbuf = inputs.guarded_buffer(M * N, poison, dtype=out).to(dev)
    sdg.gemm_bn_reduce(a.to(dev), b_kn.to(dev), pbuf[: S * M * N].view(S, M, N),
                       cbuf[: M * N].view(M, N), kps, S)
    torch.cuda.synchronize()
    p = pbuf.cpu().numpy()
    cb = inputs.stored_bits(cbuf.cpu())
    assert np.all(p[S * M * N:].view(np.uint32) == GUARD_BITS), "a partials guard changed"
    guard_c = inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[out]))[0]
    assert np.all(cb[M * N:] == guard_c), "a guard after C changed"
    return p[: S * M * N].reshape(S, M, N), cb[: M * N].reshape(M, N)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bn_shape_sweep(sdg, shape, dtype):
    M, N, K, kps, S = shape
    print(f"case bn {dtype} M{M} N{N} K{K} kps{kps} S{S}: "
          f"{sdg.describe_bn(M, N, K, kps, S, inputs.DTYPES[dtype])}", flush=True)
    a, b = inputs.make_operands(M, N, K, dtype, seed=M * 5 + N + K * 3 + S, zero_first_row=True,
                                scale_last_row=True)
    P, cbits = run_bn(sdg, a, b, kps, S)
    C = oracle.decode(cbits, "f32")
    a64, b64 = _vals(a), _vals(b)
    RP, DP, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    ep, _ = oracle.normalized_error(P, RP, DP)
    ec, _ = oracle.normalized_error(C, RC, DC)
    print(f"  partial err {ep:.3e}, final err {ec:.3e}", flush=True)
    assert ep <= PARTIAL_TOL and ec <= FINAL_TOL[dtype]
    assert np.all(P[:, 0, :] == 0) and np.all(C[0] == 0)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(96, 320, 480, 160, 3), (32, 512, 2080, 544, 4),
                                   (512, 1024, 1024, 256, 4)], ids=lambda s: "x".join(map(str, s)))
def test_bn_exact_inputs_bitwise(sdg, shape, dtype):
    M, N, K, kps, S = shape
    a, b = inputs.exact_operands(M, N, K, dtype, seed=9 + S)
    P, cbits = run_bn(sdg, a, b, kps, S)
    a64, b64 = _vals(a), _vals(b)
    RP, _, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, _, _ = oracle.gemm_bt(a64, b64)
    np.testing.assert_array_equal(P.astype(np.float64), RP)
    np.testing.assert_array_equal(oracle.decode(cbits, "f32"), RC)


def test_bn_orientation(sdg):
    """A one-hot A picks rows of the [K,N] array: C[i,j] = B[i,j] for i < M.
    A transposed read of B would give B[j,i] instead."""
    M, N, K = 64, 128, 256
    a = torch.eye(M, K, dtype=torch.bfloat16)
    _, b = inputs.make_operands(M, N, K, "bf16", seed=4)   # b is [N,K]; stored B is b^T
    P, cbits = run_bn(sdg, a, b, 128, 2)
    want = b.T[:M].to(torch.float32).numpy()                # stored [K,N] rows 0..M-1
    np.testing.assert_array_equal(oracle.decode(cbits, "f32"), want)
    assert np.all(P[1] == 0)


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_bn_typed_output(sdg, out):
    M, N, K, kps, S = 96, 512, 2048, 512, 4
    a, b = inputs.make_operands(M, N, K, "bf16", seed=31)
    _, cbits = run_bn(sdg, a, b, kps, S, out=out)
    RC, DC, _ = oracle.gemm_bt(_vals(a), _vals(b))
    err, _ = oracle.normalized_error(oracle.decode(cbits, out), RC, DC)
    assert err <= FINAL_TOL[out]


@pytest.mark.parametrize("name", ["bf16_m96_n512_k2048_s4", "bf16_m256_n1024_k2048_s2",
                                  "f16_m32_n512_k2080_s4", "f32_m32_n64_k64_s2"])
@pytest.mark.parametrize("poison", ["seven", "nan"])
def test_bn_workloads(sdg, name, poison):
    w = inputs.WORKLOADS[name]
    a, b = inputs.workload_operands(w)
    P, cbits = run_bn(sdg, a, b, w.kps, w.splits, poison=poison)
    a64, b64 = _vals(a), _vals(b)
    RP, DP, _ = oracle.splitk_partials(a64, b64, w.kps, w.splits)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    assert oracle.normalized_error(P, RP, DP)[0] <= PARTIAL_TOL
    assert oracle.normalized_error(oracle.decode(cbits, "f32"), RC, DC)[0] <= FINAL_TOL[w.dtype]


@pytest.mark.parametrize("poison", ["seven", "nan"])
def test_bn_largest_workload_full_parity(sdg, poison):
    """2048x4096x4096 in 8 splits with B stored [K,N] (its own large-tile
    kernel, streaming slab stores): every partial and every element of C
    against the binary64 reference, slab by slab, poisoned outputs, guards."""
    w = inputs.WORKLOADS[LARGEST]
    print(f"case {w.name} [K,N] poison={poison}", flush=True)
    a, b, RP, DP, RC, DC = largest_reference()
    P, cbits = run_bn(sdg, a, b, w.kps, w.splits, poison=poison)
    worst = 0.0
    for s in range(w.splits):
        ep, _ = oracle.normalized_error(P[s], RP[s], DP[s])
        worst = max(worst, ep)
        assert ep <= PARTIAL_TOL, f"slab {s}: partial error {ep}"
    ec, _ = oracle.normalized_error(oracle.decode(cbits, "f32"), RC, DC)
    print(f"  partial err {worst:.3e}, final err {ec:.3e}", flush=True)
    assert ec <= FINAL_TOL["bf16"]
