"""GPU parity: the HIP kernels, called through the C ABI, against the
binary64 reference (oracle/).

Acceptance follows the pages ("Aligned shared rows for pipelined NAX on
CUDA", section "Contract and correctness"; "Wider consecutive-weight NAX
GEMM", sections "Launch contract and correctness" and "Performance
method"): every partial within 1e-4 and the final output within 1e-4 (F32
inputs), 2e-3 (F16) or 2e-2 (BF16), the error being |gpu - ref| divided by
the sum of |products| behind the reference value (exact zero required where
that sum is zero); outputs poisoned before the call (7.0, and separately a
quiet NaN so that any element left unwritten fails); 64 trailing guard
elements at 11.0 that must come back bit-for-bit.
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


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


def _say(msg):
    print(msg, flush=True)


def _vals(t):
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


class Run:
    """One GEMM + slab sum on the GPU with guarded, poisoned outputs."""

    def __init__(self, sdg, a, b, kps, S, poison="seven", separate=False, stream=None):
        dev = torch.device("cuda:0")
        self.M, self.K = a.shape
        self.N = b.shape[0]
        self.S = S
        n_p, n_c = S * self.M * self.N, self.M * self.N
        self.pbuf = inputs.guarded_buffer(n_p, poison).to(dev)
        self.cbuf = inputs.guarded_buffer(n_c, poison).to(dev)
        P = self.pbuf[:n_p].view(S, self.M, self.N)
        C = self.cbuf[:n_c].view(self.M, self.N)
        ad, bd = a.to(dev), b.to(dev)
        if separate:
            sdg.gemm_bt(ad, bd, P, kps, S, stream=stream)
            sdg.reduce(P, C, S, stream=stream)
        else:
            sdg.gemm_bt_reduce(ad, bd, P, C, kps, S, stream=stream)
        torch.cuda.synchronize()
        self.p_all = self.pbuf.cpu().numpy()
        self.c_all = self.cbuf.cpu().numpy()
        self.P = self.p_all[:n_p].reshape(S, self.M, self.N)
        self.C = self.c_all[:n_c].reshape(self.M, self.N)

    def guards_intact(self):
        return (np.all(self.p_all[-inputs.GUARD_COUNT:].view(np.uint32) == GUARD_BITS) and
                np.all(self.c_all[-inputs.GUARD_COUNT:].view(np.uint32) == GUARD_BITS))


def check_against_oracle(sdg, a, b, kps, S, dtype, poison="seven", separate=False):
    a64, b64 = _vals(a), _vals(b)
    RP, DP, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    run = Run(sdg, a, b, kps, S, poison=poison, separate=separate)
    ep, ip = oracle.normalized_error(run.P, RP, DP)
    ec, ic = oracle.normalized_error(run.C, RC, DC)
    _say(f"  partial err {ep:.3e} at {np.unravel_index(max(ip, 0), RP.shape)}, "
         f"final err {ec:.3e} at {np.unravel_index(max(ic, 0), RC.shape)}")
    assert run.guards_intact(), "a trailing guard changed"
    assert ep <= PARTIAL_TOL, f"partial error {ep}"
    assert ec <= FINAL_TOL[dtype], f"final error {ec}"
    return run, (RP, DP, RC, DC)


# The measured workloads except the largest (checked by sampling below).
SMALL_WORKLOADS = [n for n, w in inputs.WORKLOADS.items() if w.M * w.N * w.K <= 2**31]


@pytest.mark.parametrize("name", SMALL_WORKLOADS)
@pytest.mark.parametrize("poison", ["seven", "nan"])
def test_workload_full_parity(sdg, name, poison):
    w = inputs.WORKLOADS[name]
    _say(f"case {name} poison={poison}")
    a, b = inputs.workload_operands(w)
    run, _ = check_against_oracle(sdg, a, b, w.kps, w.splits, w.dtype, poison=poison)
    if w.zero_first_row:
        assert np.all(run.P[:, 0, :] == 0) and np.all(run.C[0] == 0)


# Ten shapes x three dtypes: a single tile, non-square, a short final split,
# odd tile counts, long K, skinny, larger, and the measured shapes.
TEN_SHAPES = [
    (32, 64, 32, 32, 1),
    (64, 192, 256, 128, 2),
    (32, 512, 2080, 544, 4),
    (96, 320, 480, 160, 3),
    (32, 64, 8192, 2048, 4),
    (32, 512, 2048, 512, 4),
    (512, 1024, 1024, 512, 2),
    (96, 512, 2048, 512, 4),
    (256, 512, 2048, 1024, 2),
    (256, 1024, 2048, 1024, 2),
]
EXTRA_SHAPES = [
    (64, 128, 1056, 1024, 2),   # final split of 32
    (96, 512, 512, 128, 4),     # short K
    (64, 128, 2048, 32, 64),    # 64 splits of 32
    (160, 192, 608, 96, 7),     # five row blocks, seven splits, final split 32
    (32, 64, 64, 64, 1),        # one split
    (256, 512, 2048, 512, 4),   # the pages' 256x512x2048 row at four splits
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", TEN_SHAPES + EXTRA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shape_sweep(sdg, shape, dtype):
    M, N, K, kps, S = shape
    _say(f"case {dtype} M{M} N{N} K{K} kps{kps} S{S}")
    a, b = inputs.make_operands(M, N, K, dtype, seed=M * 7 + N * 3 + K + S, zero_first_row=True,
                                scale_last_row=True)
    run, _ = check_against_oracle(sdg, a, b, kps, S, dtype)
    assert np.all(run.P[:, 0, :] == 0) and np.all(run.C[0] == 0)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(32, 64, 64, 32, 2), (96, 320, 480, 160, 3),
                                   (32, 512, 2080, 544, 4), (256, 1024, 2048, 1024, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_exact_inputs_bitwise(sdg, shape, dtype):
    """Entries j/8 make every F32 sum exact in any order: partials and C must
    equal the reference bit for bit."""
    M, N, K, kps, S = shape
    _say(f"case exact {dtype} M{M} N{N} K{K} kps{kps} S{S}")
    a, b = inputs.exact_operands(M, N, K, dtype, seed=5 + S)
    a64, b64 = _vals(a), _vals(b)
    RP, _, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, _, _ = oracle.gemm_bt(a64, b64)
    run = Run(sdg, a, b, kps, S, poison="nan")
    assert run.guards_intact()
    np.testing.assert_array_equal(run.P.astype(np.float64), RP)
    np.testing.assert_array_equal(run.C.astype(np.float64), RC)


def test_closed_forms_on_gpu(sdg):
    """All-ones operands give each split's length (pins the last-split cut);
    a one-hot A gives C = B^T on the leading block (pins orientation)."""
    M, N, K, kps, S = 32, 512, 2080, 544, 4
    a = torch.ones(M, K, dtype=torch.float16)
    b = torch.ones(N, K, dtype=torch.float16)
    run = Run(sdg, a, b, kps, S, poison="nan")
    for s, length in enumerate([544, 544, 544, 448]):
        assert np.all(run.P[s] == length)
    assert np.all(run.C == K)
    M, N, K = 64, 128, 256
    a = torch.eye(M, K, dtype=torch.bfloat16)
    _, b = inputs.make_operands(M, N, K, "bf16", seed=3)
    run = Run(sdg, a, b, 128, 2, poison="nan")
    want = b[:, :M].to(torch.float32).T.numpy()
    np.testing.assert_array_equal(run.C, want)
    np.testing.assert_array_equal(run.P[0], want)
    assert np.all(run.P[1] == 0)
    # One-hot B (B[j,k] = [k == j], K >= N): C[i,j] = A[i,j], pinning the
    # row-major orientation of A and of the output.
    M, N, K = 96, 128, 256
    a, _ = inputs.make_operands(M, N, K, "f16", seed=8)
    b = torch.eye(N, K, dtype=torch.float16)
    run = Run(sdg, a, b, 128, 2, poison="nan")
    np.testing.assert_array_equal(run.C, a[:, :N].to(torch.float32).numpy())
    np.testing.assert_array_equal(run.P[0], a[:, :N].to(torch.float32).numpy())
    assert np.all(run.P[1] == 0)


def test_row_scaled_by_four_is_exactly_four_times(sdg):
    M, N, K, kps, S = 64, 256, 1024, 512, 2
    a, b = inputs.make_operands(M, N, K, "bf16", seed=8)
    a[5] = a[9] * 4
    run = Run(sdg, a, b, kps, S)
    np.testing.assert_array_equal(run.P[:, 5, :], 4 * run.P[:, 9, :])
    np.testing.assert_array_equal(run.C[5], 4 * run.C[9])


def test_repeated_calls_are_bitwise_identical(sdg):
    w = inputs.WORKLOADS[inputs.HEADLINE]
    a, b = inputs.workload_operands(w)
    r1 = Run(sdg, a, b, w.kps, w.splits)
    r2 = Run(sdg, a, b, w.kps, w.splits, poison="nan")
    assert np.array_equal(r1.P.view(np.uint32), r2.P.view(np.uint32))
    assert np.array_equal(r1.C.view(np.uint32), r2.C.view(np.uint32))


def test_separate_calls_match_fused_call(sdg):
    w = inputs.WORKLOADS["f16_m32_n512_k2080_s4"]
    a, b = inputs.workload_operands(w)
    r1 = Run(sdg, a, b, w.kps, w.splits)
    r2 = Run(sdg, a, b, w.kps, w.splits, separate=True)
    assert np.array_equal(r1.P.view(np.uint32), r2.P.view(np.uint32))
    assert np.array_equal(r1.C.view(np.uint32), r2.C.view(np.uint32))


def test_runs_on_a_side_stream(sdg):
    w = inputs.WORKLOADS["bf16_m96_n512_k2048_s4"]
    a, b = inputs.workload_operands(w)
    ref = Run(sdg, a, b, w.kps, w.splits)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        got = Run(sdg, a, b, w.kps, w.splits, poison="nan", stream=side)
    assert np.array_equal(ref.C.view(np.uint32), got.C.view(np.uint32))


def test_graph_replays_match_eager(sdg):
    """The chain captured into a HIP graph and replayed several times, with
    eager work and synchronisation in between; every replay must match."""
    w = inputs.WORKLOADS[inputs.HEADLINE]
    a, b = inputs.workload_operands(w)
    eager = Run(sdg, a, b, w.kps, w.splits)
    dev = torch.device("cuda:0")
    ad, bd = a.to(dev), b.to(dev)
    P = torch.empty(w.splits, w.M, w.N, device=dev)
    C = torch.empty(w.M, w.N, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sdg.gemm_bt_reduce(ad, bd, P, C, w.kps, w.splits)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            sdg.gemm_bt_reduce(ad, bd, P, C, w.kps, w.splits)
    for rep in range(4):
        P.fill_(float("nan"))
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), eager.C.view(np.uint32)), rep
        assert np.array_equal(P.cpu().numpy().view(np.uint32), eager.P.view(np.uint32)), rep


@pytest.mark.parametrize("poison", ["seven", "nan"])
def test_largest_workload_full_parity(sdg, poison):
    """The 2048x4096x4096, 8-split workload in the configuration the
    benchmark times (the large-tile kernel with streaming slab stores, then
    the streaming slab sum): every partial and every element of C against
    the binary64 reference, slab by slab, with the outputs poisoned (7.0,
    then a quiet NaN) and the guards checked."""
    w = inputs.WORKLOADS[LARGEST]
    _say(f"case {w.name} poison={poison} ({sdg.describe(w.M, w.N, w.K, w.kps, w.splits, torch.bfloat16)})")
    a, b, RP, DP, RC, DC = largest_reference()
    run = Run(sdg, a, b, w.kps, w.splits, poison=poison)
    assert run.guards_intact(), "a trailing guard changed"
    worst = 0.0
    for s in range(w.splits):
        ep, ip = oracle.normalized_error(run.P[s], RP[s], DP[s])
        worst = max(worst, ep)
        assert ep <= PARTIAL_TOL, f"slab {s}: partial error {ep} at {np.unravel_index(ip, RP[s].shape)}"
    ec, ic = oracle.normalized_error(run.C, RC, DC)
    _say(f"  partial err {worst:.3e}, final err {ec:.3e} at {np.unravel_index(max(ic, 0), RC.shape)}")
    assert ec <= FINAL_TOL["bf16"], f"final error {ec}"
    if poison == "seven":
        # Elements equal to the poison are allowed only where the reference is
        # within tolerance of it (the NaN pass proves every element written).
        left = run.C == np.float32(inputs.POISON_VALUE)
        assert np.all(np.abs(RC[left] - inputs.POISON_VALUE) <= FINAL_TOL["bf16"] * DC[left])


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 8, 13])
def test_reduce_alone(sdg, S):
    """The slab sum alone on random F32 slabs: within the F32 rounding of an
    S-term sum, (S-1) * 2^-24 of the sum of |values|; bit-exact on values
    whose sums are exact."""
    M, N = 96, 320
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(S)
    slabs = torch.randn(S, M, N, generator=gen) * 3
    cbuf = inputs.guarded_buffer(M * N, "nan").to(dev)
    sdg.reduce(slabs.to(dev), cbuf[: M * N].view(M, N), S)
    torch.cuda.synchronize()
    got = cbuf.cpu().numpy()
    ref, D, _ = oracle.slab_sum(slabs.numpy())
    err, _ = oracle.normalized_error(got[: M * N], ref, D)
    assert err <= max(S - 1, 0) * 2.0**-24 * 1.0001
    assert np.all(got[M * N:].view(np.uint32) == GUARD_BITS)
    ints = torch.randint(-1000, 1000, (S, M, N), generator=gen).float()
    C = torch.empty(M, N, device=dev)
    sdg.reduce(ints.to(dev), C, S)
    ref, _, _ = oracle.slab_sum(ints.numpy())
    np.testing.assert_array_equal(C.cpu().numpy().astype(np.float64), ref)


def test_error_statuses_with_real_buffers(sdg):
    """Misaligned pointers and overlapping outputs are rejected (nothing is
    launched), with real device memory behind every pointer."""
    dev = torch.device("cuda:0")
    M, N, K, kps, S = 64, 128, 256, 128, 2
    pool = torch.zeros(1 << 20, dtype=torch.float32, device=dev)  # 4 MiB
    base = pool.data_ptr()
    A, B, P, C = base, base + (1 << 16), base + (1 << 17), base + (1 << 19)
    call = lambda *a: sdg.raw_call("splitk_gemm_bt_reduce", *a)  # noqa: E731
    bf = inputs.DTYPE_CODES["bf16"]
    assert call(A + 4, B, P, C, M, N, K, kps, S, bf, None) == 6
    assert call(A, B, P + 8, C, M, N, K, kps, S, bf, None) == 6
    assert call(A, B, A, C, M, N, K, kps, S, bf, None) == 5
    assert call(A, B, P, P + 4096, M, N, K, kps, S, bf, None) == 5
    assert sdg.raw_call("splitk_reduce", P, P + 1024, S, M, N, None) == 5
    assert sdg.raw_call("splitk_gemm_bt", A, B, B, M, N, K, kps, S, bf, None) == 5
    torch.cuda.synchronize()
    assert torch.count_nonzero(pool).item() == 0  # nothing ran
    with pytest.raises(sdg.SplitKError):
        a = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
        b = torch.zeros(N, K, dtype=torch.bfloat16, device=dev)
        sdg.gemm_bt(a, b, torch.zeros(3, M, N, device=dev), kps, 3)


@pytest.mark.parametrize("S,M,N", [(2, 2048, 2048), (3, 2048, 2048), (8, 2048, 2048), (11, 2048, 2048),
                                   (13, 2048, 2048), (4, 4096, 4096)])
def test_reduce_alone_large_plane(sdg, S, M, N):
    """A plane large enough for the several-words-per-lane launch: sums of
    small integers are exact, so C must equal the reference bit for bit.
    The last two cases hold more than 192 MiB of slabs, which the pass reads
    with streaming loads (one of them in batches of eight slabs)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(100 + S)
    ints = torch.randint(-1000, 1000, (S, M, N), generator=gen).float()
    cbuf = inputs.guarded_buffer(M * N, "nan").to(dev)
    sdg.reduce(ints.to(dev), cbuf[: M * N].view(M, N), S)
    torch.cuda.synchronize()
    got = cbuf.cpu().numpy()
    ref, _, _ = oracle.slab_sum(ints.numpy())
    np.testing.assert_array_equal(got[: M * N].astype(np.float64), ref.ravel())
    assert np.all(got[M * N:].view(np.uint32) == GUARD_BITS)


# ------------------------------------------------ typed final output
# The F32 slab sum rounded to F16 or BF16 (nearest, ties to even); checked
# with the pages' final-output tolerances for that type, and bit for bit
# where every sum is exact (then the result is the oracle's encoding of the
# exact value).

GUARD16 = {"f16": np.float16(inputs.GUARD_VALUE).view(np.uint16),
           "bf16": np.uint16(torch.tensor([inputs.GUARD_VALUE]).to(torch.bfloat16)
                             .view(torch.int16).item() & 0xFFFF)}


def _typed_run(sdg, a, b, kps, S, out):
    dev = torch.device("cuda:0")
    M, N = a.shape[0], b.shape[0]
    P = torch.empty(S, M, N, device=dev)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    sdg.gemm_bt_reduce(a.to(dev), b.to(dev), P, cbuf[: M * N].view(M, N), kps, S)
    torch.cuda.synchronize()
    bits = inputs.stored_bits(cbuf.cpu())
    assert np.all(bits[M * N:] == GUARD16[out]), "a trailing guard changed"
    return bits[: M * N].reshape(M, N)


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("name", ["bf16_m96_n512_k2048_s4", "bf16_m256_n1024_k2048_s2",
                                  "f16_m32_n512_k2080_s4", "f32_m32_n64_k64_s2"])
def test_typed_output_parity(sdg, name, out):
    w = inputs.WORKLOADS[name]
    a, b = inputs.workload_operands(w)
    bits = _typed_run(sdg, a, b, w.kps, w.splits, out)
    RC, DC, _ = oracle.gemm_bt(_vals(a), _vals(b))
    got = oracle.decode(bits, out)
    assert not np.isnan(got).any()
    err, _ = oracle.normalized_error(got, RC, DC)
    _say(f"  typed {out} final err {err:.3e}")
    assert err <= FINAL_TOL[out]


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_typed_output_exact_inputs_bitwise(sdg, dtype, out):
    M, N, K, kps, S = 96, 320, 480, 160, 3
    a, b = inputs.exact_operands(M, N, K, dtype, seed=21)
    bits = _typed_run(sdg, a, b, kps, S, out)
    RC, _, _ = oracle.gemm_bt(_vals(a), _vals(b))
    np.testing.assert_array_equal(bits, oracle.encode(RC, out))


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("S", [1, 3, 8, 11])
@pytest.mark.parametrize("M,N", [(96, 320), (2048, 2048)])
def test_typed_reduce_alone_bitwise(sdg, out, S, M, N):
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(S + M)
    slabs = torch.randint(-4000, 4000, (S, M, N), generator=gen).float().div_(64)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    sdg.reduce(slabs.to(dev), cbuf[: M * N].view(M, N), S)
    torch.cuda.synchronize()
    bits = inputs.stored_bits(cbuf.cpu())
    ref, _, _ = oracle.slab_sum(slabs.numpy())   # exact: multiples of 1/64 well inside F32
    np.testing.assert_array_equal(bits[: M * N], oracle.encode(ref, out).ravel())
    assert np.all(bits[M * N:] == GUARD16[out])


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("S,M,N", [(13, 2048, 2048), (4, 4096, 4096)])
def test_typed_reduce_streaming_bitwise(sdg, out, S, M, N):
    """More than 192 MiB of slabs: streaming loads and streaming 8-byte
    stores of the rounded sums (one case in batches of eight slabs)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(S + M + 7)
    slabs = torch.randint(-4000, 4000, (S, M, N), generator=gen).float().div_(64)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    sdg.reduce(slabs.to(dev), cbuf[: M * N].view(M, N), S)
    torch.cuda.synchronize()
    bits = inputs.stored_bits(cbuf.cpu())
    ref, _, _ = oracle.slab_sum(slabs.numpy())
    np.testing.assert_array_equal(bits[: M * N], oracle.encode(ref, out).ravel())
    assert np.all(bits[M * N:] == GUARD16[out])
