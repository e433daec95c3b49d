"""GPU: splitk_gemm_bt_auto_noalloc, the automatic-split product with its
slabs in the library's static device array, against splitk_gemm_bt_auto
with a caller workspace (same choice, same kernels: C equal bit for bit) and
against the binary64 reference within the pages' final-output tolerances
("Aligned shared rows for pipelined NAX on CUDA", section "Contract and
correctness": F32 1e-4, F16 2e-3, BF16 2e-2).  Two calls in a row, the
second on a smaller problem, so the second reads only what it wrote over the
first's leftovers; guards after C; a problem whose slabs would not fit the
array is refused before anything runs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

FINAL_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}
STATIC_FLOATS = 16 << 20


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _c_run(sdg, fn, a, b, out):
    """C (stored bits, guards checked) from one call of `fn` into a
    NaN-poisoned, guarded buffer."""
    dev = torch.device("cuda:0")
    M, N = a.shape[0], b.shape[0]
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    fn(a.to(dev), b.to(dev), cbuf[: M * N].view(M, N))
    torch.cuda.synchronize()
    bits = inputs.stored_bits(cbuf.cpu())
    guard = inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[out]))[0]
    assert np.all(bits[M * N:] == guard), "a guard after C changed"
    return bits[: M * N].reshape(M, N)


# (M, N, K, input dtype, output dtype): each needs slabs (more than one
# split, or a rounded output); the second call of each pair is smaller.
PAIRS = [
    ((256, 1024, 8192, "bf16", "f32"), (96, 512, 4096, "bf16", "f32")),
    ((512, 1024, 2048, "bf16", "bf16"), (32, 256, 1024, "f16", "f16")),
    ((96, 1536, 12288, "f32", "f32"), (64, 128, 2048, "f32", "bf16")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "-".join("x".join(map(str, c)) for c in p))
def test_noalloc_matches_workspace_call(sdg, pair):
    dev = torch.device("cuda:0")
    for M, N, K, dt, out in pair:
        kps, S, need = sdg.choose_splits(M, N, K, inputs.DTYPES[dt], inputs.DTYPES[out])
        print(f"case noalloc M{M} N{N} K{K} {dt}->{out}: splits {S} kps {kps} slabs {need}", flush=True)
        assert 0 < need <= STATIC_FLOATS, "the case must use the static slab array"
        a, b = inputs.make_operands(M, N, K, dt, seed=M + N + K, zero_first_row=True, scale_last_row=True)
        W = torch.empty(need, device=dev)
        ref_bits = _c_run(sdg, lambda A, B, C: sdg.gemm_bt_auto(A, B, C, workspace=W), a, b, out)
        got_bits = _c_run(sdg, sdg.gemm_bt_auto_noalloc, a, b, out)
        np.testing.assert_array_equal(got_bits, ref_bits)
        RC, DC, _ = oracle.gemm_bt(oracle.decode(inputs.stored_bits(a), dt),
                                   oracle.decode(inputs.stored_bits(b), dt))
        err, _ = oracle.normalized_error(oracle.decode(got_bits, out), RC, DC)
        tol = FINAL_TOL[out] if out != "f32" else FINAL_TOL[dt]
        print(f"  final err {err:.3e} (tolerance {tol})", flush=True)
        assert err <= tol


def test_noalloc_direct_path(sdg):
    """One split with an F32 C needs no slabs: the GEMM writes C directly."""
    M, N, K = 256, 1024, 2048
    kps, S, need = sdg.choose_splits(M, N, K, torch.bfloat16)
    if need != 0:
        pytest.skip("this shape no longer takes the direct path")
    a, b = inputs.make_operands(M, N, K, "bf16", seed=9)
    ref = _c_run(sdg, lambda A, B, C: sdg.gemm_bt_auto(A, B, C), a, b, "f32")
    got = _c_run(sdg, sdg.gemm_bt_auto_noalloc, a, b, "f32")
    np.testing.assert_array_equal(got, ref)


def test_noalloc_refuses_slabs_beyond_the_array(sdg):
    """4096x8192 outputs rounded to BF16 need at least 32 Mi slab elements,
    twice the array: refused with SPLITK_ERR_SCRATCH and nothing runs (every
    buffer is full-sized, so nothing could land out of bounds either)."""
    dev = torch.device("cuda:0")
    M, N, K = 4096, 8192, 1024
    kps, S, need = sdg.choose_splits(M, N, K, torch.bfloat16, torch.bfloat16)
    assert need > STATIC_FLOATS
    A = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
    B = torch.zeros(N, K, dtype=torch.bfloat16, device=dev)
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sdg.SplitKError) as e:
        sdg.gemm_bt_auto_noalloc(A, B, C)
    assert e.value.status == 11
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)
