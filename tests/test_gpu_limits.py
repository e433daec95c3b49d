"""Sizes at the limits of the C ABI, on the GPU.

The boundary accepts a problem only while every buffer holds fewer than 2^31
elements: splits*M*N partials, M*N outputs, M*K and N*K operand elements.
Each case below comes within a few thousand elements of one or more of those
limits, so an offset computed in 32 bits anywhere in a kernel would wrap and
land on the wrong element (or outside the buffer).  The cases take the kernel
families the planner uses at such sizes: the persistent 256x256 kernel, the
one-tile 256x256 kernel of B stored [K,N], both with narrowed last column
tiles too, 256x128 tiles with a 64-column tail, the skinny LDS-DMA kernel on
a million workgroups, and the
register-staged skinny kernel on 32 splits of a million k each.

Operands are exact products of seeded small integers, A[i,k] = a[i]*u[k] and
B[j,k] = b[j]*v[k] (``inputs.product_factors``).  Then every partial is
a[i]*b[j]*w[s], w[s] being the sum of u[k]*v[k] over split s's k range, and
every output is a[i]*b[j] times the sum of all w[s] (the definition of the
partials and of the final output: "Aligned shared rows for pipelined NAX on
CUDA", section "Contract and correctness").  Each case first checks that
every value, and every partial sum in any order, is an integer below 2^24,
so F32 accumulation is exact and the whole of every slab and of C must equal
the closed form.  The closed form is pinned to the binary64 reference on small
shapes (the CPU test at the end).  Outputs start as quiet NaN, so an element
left unwritten fails, with 64 guard elements at 11.0 after each buffer.

One further case runs random (full-rank) operands at the persistent kernel's
near-limit shape and compares sampled outputs, the buffer corners among them,
with the reference at the pages' tolerances.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

GUARD_BITS = int(np.float32(inputs.GUARD_VALUE).view(np.int32))
LIMIT = 2**31
EXACT = 2**24

# (name, M, N, K, k_per_split, splits, dtype, B layout, kernel the planner must pick)
CASES = [
    # splits*M*N = 2,147,352,576: the persistent kernel, 32,766 tiles on 256 workgroups
    ("persistent", 11008, 97536, 256, 128, 2, "bf16", "nk", "persistent"),
    ("persistent_f32", 11008, 97536, 256, 128, 2, "f32", "nk", "persistent"),
    # the same with B stored [K,N]: one 256x256 tile per workgroup
    ("kn", 11008, 97536, 256, 128, 2, "bf16", "kn", "tiled bm256 bn256"),
    # splits*M*N = 2,145,386,496: the persistent kernel, the last column tile 192 wide
    ("persistent_tail", 8192, 65472, 128, 32, 4, "bf16", "nk", "persistent"),
    # splits*M*N = 2,136,997,888: 256x128 tiles (the last round of 256x256
    # ones would be half full), the last column tile 64 wide
    ("tail", 8192, 65216, 128, 32, 4, "bf16", "nk", "tiled bm256 bn128"),
    # splits*M*N = M*K = 2,147,479,552: 1,048,574 workgroups
    ("tall", 16777184, 64, 128, 64, 2, "bf16", "nk", "wavekdma"),
    # N*K = 2,147,481,600 (rows of 64 MiB): 32 splits of 2^20
    ("long_k", 32, 64, 33554400, 1048576, 32, "bf16", "nk", "wavek "),
]


def closed_form(factors, K: int, kps: int, splits: int):
    """(w, wc): w[s] = sum of u[k]*v[k] over split s's k range (int64), and
    wc = sum of w; the partial [s,i,j] is a[i]*b[j]*w[s], the output a[i]*b[j]*wc."""
    _, _, u, v = factors
    uv = (u * v).numpy()
    w = np.array([int(uv[s * kps:min((s + 1) * kps, K)].sum()) for s in range(splits)], dtype=np.int64)
    return w, int(w.sum())


def _exactness_bound(factors, K: int, kps: int, splits: int) -> tuple[int, int]:
    """Largest magnitude any partial sum can take inside a split (in any
    order), and largest magnitude of the ascending-s running sum of slabs."""
    a, b, u, v = factors
    ab = int(a.abs().max()) * int(b.abs().max())
    nz = (u * v).abs().numpy()
    inside = max(int(nz[s * kps:min((s + 1) * kps, K)].sum()) for s in range(splits)) * ab
    w, _ = closed_form(factors, K, kps, splits)
    running = int(np.abs(np.cumsum(w)).max()) * ab
    return inside, running


def _guarded(n: int, dev) -> torch.Tensor:
    buf = torch.empty(n + inputs.GUARD_COUNT, dtype=torch.float32, device=dev)
    buf[:n].view(torch.int32).fill_(inputs.NAN_POISON_BITS)
    buf[n:].fill_(inputs.GUARD_VALUE)
    return buf


def _guards_intact(buf: torch.Tensor) -> bool:
    tail = buf[-inputs.GUARD_COUNT:].cpu().view(torch.int32)
    return bool((tail == GUARD_BITS).all())


def _compare_plane(got_dev: torch.Tensor, af: torch.Tensor, bf: torch.Tensor, scale: int, what: str):
    """Every element of the [M,N] device plane against a[i]*b[j]*scale, exactly,
    in row blocks of about 16 M elements.  The expected values are integers
    below 2^24 (checked by the caller), so F32 holds them and their products
    exactly."""
    M, N = got_dev.shape
    rows = max(1, (1 << 24) // N)
    for r0 in range(0, M, rows):
        got = got_dev[r0:r0 + rows].cpu()
        exp = torch.outer(af[r0:r0 + rows], bf) * float(scale)
        if not torch.equal(got, exp):
            bad = (got != exp).nonzero()[0].tolist()
            i, j = r0 + bad[0], bad[1]
            raise AssertionError(f"{what}[{i},{j}] = {got[bad[0], bad[1]].item()!r}, "
                                 f"expected {exp[bad[0], bad[1]].item()!r}")


@pytest.fixture(scope="module")
def sdg(hip_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return hip_lib


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_limit_sizes_exact(sdg, case):
    name, M, N, K, kps, S, dtype, layout, kernel = case
    assert S * M * N < LIMIT and M * N < LIMIT and M * K < LIMIT and N * K < LIMIT
    assert (S - 1) * kps < K <= S * kps
    code = inputs.DTYPE_CODES[dtype]
    plan = sdg.describe(M, N, K, kps, S, code) if layout == "nk" else sdg.describe_bn(M, N, K, kps, S, code)
    print(f"  {name}: {M}x{N}x{K} kps {kps} S {S} {dtype} B[{layout}]: {plan}", flush=True)
    assert kernel in plan

    factors = inputs.product_factors(M, N, K, seed=M + N + K)
    inside, running = _exactness_bound(factors, K, kps, S)
    assert inside < EXACT and running < EXACT, (inside, running)
    w, wc = closed_form(factors, K, kps, S)

    dev = torch.device("cuda:0")
    try:
        A, B = inputs.product_operands(factors, dtype, dev, b_layout=layout)
        pbuf, cbuf = _guarded(S * M * N, dev), _guarded(M * N, dev)
        P = pbuf[:S * M * N].view(S, M, N)
        C = cbuf[:M * N].view(M, N)
        if layout == "nk":
            sdg.gemm_bt_reduce(A, B, P, C, kps, S)
        else:
            sdg.gemm_bn_reduce(A, B, P, C, kps, S)
        torch.cuda.synchronize()
        del A, B
        assert _guards_intact(pbuf), "a guard after the partials changed"
        assert _guards_intact(cbuf), "a guard after C changed"
        af, bf = factors[0].to(torch.float32), factors[1].to(torch.float32)
        for s in range(S):
            _compare_plane(P[s], af, bf, int(w[s]), f"partials[{s}]")
        _compare_plane(C, af, bf, wc, "C")
    finally:
        torch.cuda.synchronize()
        A = B = P = C = pbuf = cbuf = None
        torch.cuda.empty_cache()


@pytest.mark.gpu
def test_limit_size_random_sampled(sdg):
    """Full-rank operands at the persistent kernel's near-limit shape; the
    reference at rows and columns on both sides of tile boundaries near both
    ends of the buffers, and at seeded random ones."""
    M, N, K, kps, S = 11008, 97536, 256, 128, 2
    a, b = inputs.make_operands(M, N, K, "bf16", seed=4242)
    rng = np.random.default_rng(4242)
    rows = sorted(set([0, 1, 255, 256, M // 2, M - 257, M - 256, M - 2, M - 1] +
                      rng.integers(0, M, 12).tolist()))
    cols = sorted(set([0, 1, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 2, N - 1] +
                      rng.integers(0, N, 12).tolist()))
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    rr, cc = rr.ravel(), cc.ravel()
    a64 = oracle.decode(inputs.stored_bits(a), "bf16")
    b64 = oracle.decode(inputs.stored_bits(b), "bf16")
    RP, DP, RC, DC = oracle.sampled(a64, b64, kps, S, rr, cc)

    dev = torch.device("cuda:0")
    try:
        pbuf, cbuf = _guarded(S * M * N, dev), _guarded(M * N, dev)
        P = pbuf[:S * M * N].view(S, M, N)
        C = cbuf[:M * N].view(M, N)
        sdg.gemm_bt_reduce(a.to(dev), b.to(dev), P, C, kps, S)
        torch.cuda.synchronize()
        assert _guards_intact(pbuf) and _guards_intact(cbuf)
        assert not bool(torch.isnan(P).any()) and not bool(torch.isnan(C).any()), "an output left unwritten"
        ri, ci = torch.tensor(rr, device=dev), torch.tensor(cc, device=dev)
        gp = P[:, ri, ci].cpu().numpy().T          # [pairs, S]
        gc = C[ri, ci].cpu().numpy()
    finally:
        torch.cuda.synchronize()
        P = C = pbuf = cbuf = None
        torch.cuda.empty_cache()
    ep, _ = oracle.normalized_error(gp, RP, DP)
    ec, _ = oracle.normalized_error(gc, RC, DC)
    print(f"  {len(rr)} sampled outputs: partial err {ep:.3e}, final err {ec:.3e}", flush=True)
    assert ep <= 1e-4 and ec <= 2e-2


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,K,kps,S", [(32, 64, 96, 32, 3), (64, 128, 200, 64, 4), (32, 64, 1000, 512, 2)])
def test_closed_form_matches_reference(dtype, M, N, K, kps, S):
    """The closed form the limit cases check against equals the binary64
    reference of the same operands, element for element (CPU only)."""
    factors = inputs.product_factors(M, N, K, seed=7 + M + K)
    A, B = inputs.product_operands(factors, dtype, "cpu")
    a64 = oracle.decode(inputs.stored_bits(A), dtype)
    b64 = oracle.decode(inputs.stored_bits(B), dtype)
    RP, _, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, _, _ = oracle.gemm_bt(a64, b64)
    w, wc = closed_form(factors, K, kps, S)
    ab = np.outer(factors[0].numpy(), factors[1].numpy()).astype(np.float64)
    for s in range(S):
        assert np.array_equal(RP[s], ab * w[s]), s
    assert np.array_equal(RC, ab * wc)
    # and the [K,N] operand is the transpose of the [N,K] one
    _, Bkn = inputs.product_operands(factors, dtype, "cpu", b_layout="kn")
    assert torch.equal(Bkn, B.t())
