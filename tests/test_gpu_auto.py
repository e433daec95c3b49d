"""GPU parity of the automatic split count (splitk_gemm_bt_auto).

The pages time each shape at the split counts 1, 2, 4, 8 and 16 and keep the
fastest ("Aligned shared rows for pipelined NAX on CUDA", section
"Measurement protocol"; "Wider consecutive-weight NAX GEMM", section
"Performance method"); the library picks one of them itself.  Whatever it
picks, C must meet the final-output tolerances of "Contract and
correctness" (per input type for an F32 C, per output type for a typed C)
against the binary64 reference, be bit-identical to the explicit call with
the same geometry, and leave the guards after C and the workspace intact.
One split with an F32 C writes C straight from the GEMM (no workspace).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from conftest import LARGEST, largest_reference
from split_dense_gemm_amd import inputs

pytestmark = pytest.mark.gpu

FINAL_TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}

# (M, N, K, input type): chosen so that the picks cover one split written
# directly, typed single-split output, 2..8 splits, 16 splits (the batched
# reduce), and 16-bit splits that end in half chunks.
AUTO_SHAPES = [
    (32, 64, 64, "f32"),
    (96, 512, 2048, "bf16"),
    (256, 1024, 2048, "bf16"),
    (32, 512, 2080, "f16"),
    (32, 512, 16384, "f32"),
    (1024, 512, 8192, "bf16"),
    (512, 1024, 1024, "f16"),
    (64, 192, 4096, "bf16"),
]


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _vals(t):
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


def _guard_bits(dtype):
    return inputs.stored_bits(torch.tensor([inputs.GUARD_VALUE], dtype=inputs.DTYPES[dtype]))[0]


def _auto(sdg, a, b, out, with_workspace=False):
    """Runs the automatic path; returns (C bits, chosen geometry)."""
    dev = torch.device("cuda:0")
    M, K = a.shape
    N = b.shape[0]
    dt = inputs.DTYPES[inputs.dtype_name(a)]
    kps, S, need = sdg.choose_splits(M, N, K, dt, inputs.DTYPES[out])
    print(f"case auto M={M} N={N} K={K} {inputs.dtype_name(a)}->{out}: kps={kps} splits={S} "
          f"workspace={need}", flush=True)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    # With a need, the workspace is `need` poisoned elements followed by
    # guards; without one, either no workspace or a buffer of guards only,
    # which must come back untouched.
    wbuf = inputs.guarded_buffer(need, "nan").to(dev) if (need or with_workspace) else None
    ws = None if wbuf is None else (wbuf[:need] if need else wbuf)
    sdg.gemm_bt_auto(a.to(dev), b.to(dev), cbuf[: M * N].view(M, N), workspace=ws)
    torch.cuda.synchronize()
    cb = inputs.stored_bits(cbuf.cpu())
    assert np.all(cb[M * N:] == _guard_bits(out)), "a guard after C changed"
    if wbuf is not None:
        wb = inputs.stored_bits(wbuf.cpu())
        assert np.all(wb[need:] == _guard_bits("f32")), "a guard after the workspace changed"
    return cb[: M * N].reshape(M, N), (kps, S, need)


def _explicit(sdg, a, b, out, kps, S):
    """The same product through the explicit-geometry entry points."""
    dev = torch.device("cuda:0")
    M, N = a.shape[0], b.shape[0]
    P = torch.empty(S, M, N, device=dev)
    C = torch.empty(M, N, device=dev, dtype=inputs.DTYPES[out])
    sdg.gemm_bt_reduce(a.to(dev), b.to(dev), P, C, kps, S)
    torch.cuda.synchronize()
    if S == 1 and out == "f32":
        # One slab is the whole sum: the direct path must equal it bit for bit.
        return inputs.stored_bits(P[0].cpu())
    return inputs.stored_bits(C.cpu())


def test_shapes_cover_every_path(sdg):
    picks = set()
    for M, N, K, dt in AUTO_SHAPES:
        for out in ("f32", "bf16"):
            picks.add(sdg.choose_splits(M, N, K, inputs.DTYPES[dt], inputs.DTYPES[out])[1:])
    splits = {s for s, _ in picks}
    assert (1, 0) in picks, "no shape exercises the direct single-split path"
    assert any(s == 1 and need > 0 for s, need in picks), "no typed single-split case"
    assert any(1 < s <= 8 for s in splits) and 16 in splits, splits


@pytest.mark.parametrize("shape", AUTO_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("typed", [False, True], ids=["f32out", "typedout"])
def test_auto_parity(sdg, shape, typed):
    M, N, K, dt = shape
    out = ("bf16" if dt == "f32" else dt) if typed else "f32"
    a, b = inputs.make_operands(M, N, K, dt, seed=M + N + K, zero_first_row=True,
                                scale_last_row=True)
    bits, (kps, S, need) = _auto(sdg, a, b, out)
    got = oracle.decode(bits, out)
    assert not np.isnan(got).any(), "an element of C was left unwritten"
    RC, DC, _ = oracle.gemm_bt(_vals(a), _vals(b))
    err, idx = oracle.normalized_error(got, RC, DC)
    tol = FINAL_TOL[out] if typed else FINAL_TOL[dt]
    print(f"  final err {err:.3e} (tolerance {tol})", flush=True)
    assert err <= tol
    assert np.all(got[0] == 0), "zero first row of A must give a zero row of C"
    np.testing.assert_array_equal(bits, _explicit(sdg, a, b, out, kps, S))


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_auto_exact_inputs_bitwise(sdg, out):
    for M, N, K in ((96, 320, 480), (32, 512, 16384), (256, 1024, 1024)):
        a, b = inputs.exact_operands(M, N, K, "bf16", seed=K)
        bits, _ = _auto(sdg, a, b, out)
        RC, _, _ = oracle.gemm_bt(_vals(a), _vals(b))
        np.testing.assert_array_equal(bits, oracle.encode(RC, out))


def test_auto_direct_path_ignores_a_workspace(sdg):
    """A workspace passed where none is needed is left untouched (its guard
    region, here the whole buffer, keeps its bits)."""
    a, b = inputs.make_operands(256, 1024, 2048, "bf16", seed=5)
    kps, S, need = sdg.choose_splits(256, 1024, 2048, torch.bfloat16)
    if need != 0:
        pytest.skip("this shape no longer takes the direct path")
    bits, _ = _auto(sdg, a, b, "f32", with_workspace=True)
    RC, DC, _ = oracle.gemm_bt(_vals(a), _vals(b))
    assert oracle.normalized_error(oracle.decode(bits, "f32"), RC, DC)[0] <= FINAL_TOL["bf16"]


def test_auto_largest_workload_full(sdg):
    """The 2048x4096x4096 BF16 problem through the automatic path: every
    element of C against the binary64 reference; no NaN poison left."""
    w = inputs.WORKLOADS[LARGEST]
    a, b, _, _, RC, DC = largest_reference()
    bits, (kps, S, need) = _auto(sdg, a, b, "f32")
    got = oracle.decode(bits, "f32")
    assert not np.isnan(got).any()
    err, _ = oracle.normalized_error(got, RC, DC)
    print(f"  {w.name} auto S={S} kps={kps}: final err {err:.3e}", flush=True)
    assert err <= FINAL_TOL["bf16"]


def test_auto_workspace_too_small_launches_nothing(sdg):
    dev = torch.device("cuda:0")
    a, b = inputs.make_operands(32, 512, 16384, "bf16", seed=3)
    kps, S, need = sdg.choose_splits(32, 512, 16384, torch.bfloat16)
    assert need > 0
    C = torch.full((32, 512), 7.0, device=dev)
    W = torch.empty(need - 4, device=dev)
    with pytest.raises(sdg.SplitKError) as e:
        sdg.gemm_bt_auto(a.to(dev), b.to(dev), C, workspace=W)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)
