"""Pins for the F64 reference (oracle/), independent of the HIP path.

Each pin compares the reference with something other than itself: IEEE-754
bit patterns, torch's own decoder, exact rational arithmetic, numpy's float64
GEMM, integer arithmetic, closed forms of structured inputs and invariants of
the definition.  The last tests run the same pin suite against deliberately
wrong references (a dropped term, a shifted split, a transposed operand, a
flipped sign, swapped output indices) and require each to be caught.

Definition pinned ("Aligned shared rows for pipelined NAX on CUDA", section
"Contract and correctness"; "Wider consecutive-weight NAX GEMM", section
"Launch contract and correctness"): partials[s,i,j] = sum over
k in [s*kps, min((s+1)*kps, K)) of A[i,k]*B[j,k]; final = sum over all k.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from split_dense_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U53 = 2.0**-53


def _vals(t: torch.Tensor) -> np.ndarray:
    return oracle.decode(inputs.stored_bits(t), inputs.dtype_name(t))


def _operands(M, N, K, dtype, seed, **kw):
    a, b = inputs.make_operands(M, N, K, dtype, seed, **kw)
    return _vals(a), _vals(b)


# ---------------------------------------------------------------- decoding


def _golden_bits():
    rows = []
    with open(os.path.join(GOLDEN, "decode_bits.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            dt, bits, value = line.split()
            rows.append((dt, int(bits, 16), float.fromhex(value)))
    return rows


@pytest.mark.parametrize("dt,bits,value", _golden_bits())
def test_decode_ieee_bit_patterns(dt, bits, value):
    arr = np.array([bits], dtype=np.uint32 if dt == "f32" else np.uint16)
    got = oracle.decode(arr, dt)[0]
    assert got == value and math.copysign(1, got) == math.copysign(1, value)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_decode_matches_torch_on_random_finite_bits(dt):
    rng = np.random.default_rng(7)
    if dt == "f32":
        bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
        t = torch.from_numpy(bits.view(np.int32).copy()).view(torch.float32)
    else:
        bits = rng.integers(0, 2**16, size=20000, dtype=np.uint32).astype(np.uint16)
        t = torch.from_numpy(bits.view(np.int16).copy()).view(inputs.DTYPES[dt])
    want = t.to(torch.float64).numpy()
    got = oracle.decode(bits, dt)
    finite = np.isfinite(want)
    assert finite.sum() > 15000
    np.testing.assert_array_equal(got[finite], want[finite])
    assert np.all(np.isnan(got[np.isnan(want)]))
    assert np.array_equal(got[np.isinf(want)], want[np.isinf(want)])


# ------------------------------------------------------------ pin suite


def _fraction_products(a, b, k0, k1, i, j):
    s = Fraction(0)
    m = Fraction(0)
    for k in range(k0, k1):
        p = Fraction(a[i, k]) * Fraction(b[j, k])
        s += p
        m += abs(p)
    return s, m


def pin_bruteforce(partials_fn, full_fn):
    """Exact rational sums on tiny shapes; the binary64 result must sit within
    its own summation bound (len * 2^-53 * sum|terms|)."""
    failures = []
    for (M, N, K, kps, S, dt, seed) in [(3, 4, 8, 3, 3, "bf16", 11), (2, 5, 12, 8, 2, "f16", 12),
                                        (4, 3, 7, 7, 1, "f32", 13), (32, 64, 32, 32, 1, "bf16", 14)]:
        a, b = _operands(M, N, K, dt, seed)
        P, DP = partials_fn(a, b, kps, S)
        C, DC = full_fn(a, b)
        cells = [(i, j) for i in range(M) for j in range(N)]
        if len(cells) > 64:
            cells = cells[:: len(cells) // 64]
        for (i, j) in cells:
            for s in range(S):
                k0, k1 = s * kps, min(K, (s + 1) * kps)
                ex, em = _fraction_products(a, b, k0, k1, i, j)
                bound = (k1 - k0) * U53 * float(em) * 1.01
                if abs(P[s, i, j] - float(ex)) > bound or abs(DP[s, i, j] - float(em)) > bound:
                    failures.append(("bruteforce-partial", M, N, K, s, i, j))
            ex, em = _fraction_products(a, b, 0, K, i, j)
            bound = K * U53 * float(em) * 1.01
            if abs(C[i, j] - float(ex)) > bound or abs(DC[i, j] - float(em)) > bound:
                failures.append(("bruteforce-full", M, N, K, i, j))
    return failures


def pin_numpy_gemm(partials_fn, full_fn):
    """splits=1 and the unsplit product against numpy's float64 A @ B.T."""
    failures = []
    for (M, N, K, dt, seed) in [(32, 64, 64, "f32", 21), (64, 128, 256, "bf16", 22),
                                (96, 64, 160, "f16", 23)]:
        a, b = _operands(M, N, K, dt, seed)
        ref = a @ b.T
        D = np.abs(a) @ np.abs(b).T
        P, DP = partials_fn(a, b, K, 1)
        C, DC = full_fn(a, b)
        tol = 2 * K * U53 * D + 1e-300
        if not np.all(np.abs(P[0] - ref) <= tol):
            failures.append(("numpy-splits1", M, N, K))
        if not np.all(np.abs(C - ref) <= tol):
            failures.append(("numpy-full", M, N, K))
        if not np.all(np.abs(DC - D) <= tol) or not np.all(np.abs(DP[0] - D) <= tol):
            failures.append(("numpy-abs", M, N, K))
    return failures


def pin_exact_integers(partials_fn, full_fn):
    """Entries j/8 make every partial sum exact: compare bit-for-bit with
    integer arithmetic (64 * value is an integer)."""
    failures = []
    for (M, N, K, kps, S, dt, seed) in [(32, 64, 2080, 544, 4, "f16", 31),
                                        (64, 64, 96, 32, 3, "bf16", 32)]:
        at, bt = inputs.exact_operands(M, N, K, dt, seed)
        a, b = _vals(at), _vals(bt)
        ia = np.rint(a * 8).astype(np.int64)
        ib = np.rint(b * 8).astype(np.int64)
        P, _ = partials_fn(a, b, kps, S)
        C, _ = full_fn(a, b)
        for s in range(S):
            k0, k1 = s * kps, min(K, (s + 1) * kps)
            want = (ia[:, k0:k1] @ ib[:, k0:k1].T).astype(np.float64) / 64.0
            if not np.array_equal(P[s], want):
                failures.append(("exact-partial", M, N, K, s))
        if not np.array_equal(C, (ia @ ib.T).astype(np.float64) / 64.0):
            failures.append(("exact-full", M, N, K))
    return failures


def pin_closed_forms(partials_fn, full_fn):
    failures = []
    # All ones: every partial equals its split length; the final equals K.
    M, N, K, kps, S = 32, 64, 2080, 544, 4
    ones_a, ones_b = np.ones((M, K)), np.ones((N, K))
    P, DP = partials_fn(ones_a, ones_b, kps, S)
    for s, length in enumerate([544, 544, 544, 448]):
        if not (np.all(P[s] == length) and np.all(DP[s] == length)):
            failures.append(("ones", s))
    C, _ = full_fn(ones_a, ones_b)
    if not np.all(C == K):
        failures.append(("ones-full",))
    # One-hot A (A[i,k] = [k == i]): final C[i,j] = B[j,i]; the split holding
    # k = i carries it and every other split is zero.
    M, N, K, kps, S = 64, 64, 96, 32, 3
    a = np.eye(M, K)
    b = _operands(M, N, K, "bf16", 41)[1]
    C, _ = full_fn(a, b)
    if not np.array_equal(C, b[:, :M].T):
        failures.append(("onehot-a-full",))
    P, _ = partials_fn(a, b, kps, S)
    for s in range(S):
        want = np.zeros((M, N))
        for i in range(M):
            if s * kps <= i < (s + 1) * kps:
                want[i] = b[:, i]
        if not np.array_equal(P[s], want):
            failures.append(("onehot-a-partial", s))
    # One-hot B (B[j,k] = [k == j]): C[i,j] = A[i,j].
    M, N, K = 32, 64, 128
    a = _operands(M, N, K, "f16", 42)[0]
    b = np.eye(N, K)
    C, _ = full_fn(a, b)
    if not np.array_equal(C, a[:, :N]):
        failures.append(("onehot-b-full",))
    return failures


def pin_invariants(partials_fn, full_fn):
    failures = []
    M, N, K, kps, S = 64, 128, 1056, 1024, 2  # last split of 32
    a, b = _operands(M, N, K, "bf16", 51, zero_first_row=True, scale_last_row=True)
    P, DP = partials_fn(a, b, kps, S)
    C, DC = full_fn(a, b)
    if not (np.all(P[:, 0, :] == 0) and np.all(C[0] == 0)):
        failures.append(("zero-row",))
    if not np.all(np.abs(P.sum(axis=0) - C) <= 2 * K * U53 * DC):
        failures.append(("sum-of-slabs",))
    if not np.allclose(DP.sum(axis=0), DC, rtol=4 * K * U53, atol=0):
        failures.append(("sum-of-scales",))
    # A duplicated row scaled by 4 (a power of two) gives exactly 4x.
    a2 = a.copy()
    a2[1] = 4 * a[2]
    P2, _ = partials_fn(a2, b, kps, S)
    if not np.array_equal(P2[:, 1, :], 4 * P[:, 2, :]):
        failures.append(("scale-row",))
    return failures


PINS = [pin_bruteforce, pin_numpy_gemm, pin_exact_integers, pin_closed_forms, pin_invariants]


def _real_partials(a, b, kps, S):
    P, DP, _ = oracle.splitk_partials(a, b, kps, S)
    return P, DP


def _real_full(a, b):
    C, DC, _ = oracle.gemm_bt(a, b)
    return C, DC


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(_real_partials, _real_full) == []


# --------------------------------------------------------------- mutants
# Plausible mistakes, each written as a plain numpy reference.  Every one
# must trip at least one pin above.


def _np_partials(a, b, kps, S, start_shift=0, end_shift=0, transpose_b=False, sign_k=None,
                 swap_ij=False):
    M, K = a.shape
    N = b.shape[0]
    P = np.zeros((S, M, N))
    DP = np.zeros((S, M, N))
    for s in range(S):
        k0 = s * kps + start_shift
        k1 = min(K, (s + 1) * kps) + end_shift
        aa = a[:, k0:k1].copy()
        # transpose_b: read B's storage as if it were [K,N] (the classic layout slip)
        bsrc = b.reshape(K, N).T if transpose_b else b
        bb = bsrc[:, k0:k1]
        if sign_k is not None and k1 - k0 > sign_k:
            aa[:, sign_k] = -aa[:, sign_k]
        P[s] = aa @ bb.T
        DP[s] = np.abs(aa) @ np.abs(bb).T
        if swap_ij and M == N:
            P[s] = P[s].T
    return P, DP


def _mutant(**kw):
    def partials(a, b, kps, S):
        return _np_partials(a, b, kps, S, **kw)

    def full(a, b):
        P, DP = _np_partials(a, b, a.shape[1], 1, **kw)
        return P[0], DP[0]

    return partials, full


MUTANTS = {
    "drop-last-term": _mutant(end_shift=-1),
    "split-starts-one-late": _mutant(start_shift=1),
    "transposed-B": _mutant(transpose_b=True),
    "sign-flip-one-term": _mutant(sign_k=5),
    "swapped-output-indices": _mutant(swap_ij=True),
}


def test_numpy_twin_passes_pins():
    """The unmutated numpy twin passes, so a mutant's failure is its mutation."""
    partials, full = _mutant()
    assert all(pin(partials, full) == [] for pin in PINS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name):
    partials, full = MUTANTS[name]
    failures = [f for pin in PINS for f in pin(partials, full)]
    assert failures, f"mutant {name} passed every pin"


# ------------------------------------------------------- other functions


def test_split_geometry_rejected():
    a = np.ones((32, 64))
    b = np.ones((64, 64))
    with pytest.raises(ValueError):
        oracle.splitk_partials(a, b, 32, 3)  # third split would start at K
    with pytest.raises(ValueError):
        oracle.splitk_partials(a, b, 16, 2)  # splits do not cover K


def test_golden_split_lengths():
    with open(os.path.join(GOLDEN, "split_geometry.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            K, kps, S, lengths = line.split(maxsplit=3)
            K, kps, S = int(K), int(kps), int(S)
            want = [int(x) for x in lengths.split(",")]
            a = np.ones((32, K))
            b = np.ones((64, K))
            P, _, _ = oracle.splitk_partials(a, b, kps, S)
            assert [P[s, 0, 0] for s in range(S)] == want


def test_slab_sum_against_fsum():
    rng = np.random.default_rng(5)
    for S in (1, 2, 4, 8, 13):
        slabs = rng.standard_normal((S, 32, 64)).astype(np.float32) * np.float32(3.0)
        C, D, _ = oracle.slab_sum(slabs)
        exact = np.array([[math.fsum(slabs[:, i, j].astype(np.float64)) for j in range(64)]
                          for i in range(32)])
        assert np.all(np.abs(C - exact) <= S * U53 * D)
        assert np.array_equal(D, np.abs(slabs.astype(np.float64)).sum(axis=0)) or np.allclose(
            D, np.abs(slabs.astype(np.float64)).sum(axis=0), rtol=S * U53, atol=0)


def test_slab_sum_closed_form():
    slabs = np.full((6, 32, 64), 0.25, dtype=np.float32)
    slabs[3] = -1.5
    C, D, _ = oracle.slab_sum(slabs)
    assert np.all(C == 5 * 0.25 - 1.5) and np.all(D == 5 * 0.25 + 1.5)


def test_sampled_equals_full():
    M, N, K, kps, S = 64, 128, 1056, 1024, 2
    a, b = _operands(M, N, K, "bf16", 61)
    P, DP, _ = oracle.splitk_partials(a, b, kps, S)
    C, DC, _ = oracle.gemm_bt(a, b)
    rng = np.random.default_rng(3)
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    sp, sdp, sc, sdc = oracle.sampled(a, b, kps, S, rows, cols)
    assert np.array_equal(sp, P[:, rows, cols].T) and np.array_equal(sdp, DP[:, rows, cols].T)
    assert np.array_equal(sc, C[rows, cols]) and np.array_equal(sdc, DC[rows, cols])


def test_thread_count_does_not_change_results():
    a, b = _operands(96, 64, 512, "f16", 71)
    P1, _, t1 = oracle.splitk_partials(a, b, 128, 4, nthreads=1)
    P4, _, t4 = oracle.splitk_partials(a, b, 128, 4, nthreads=4)
    assert t1 == 1 and t4 == 4
    assert np.array_equal(P1, P4)


def test_normalized_error_rules():
    ref = np.array([1.0, 0.0, 2.0])
    den = np.array([2.0, 0.0, 4.0])
    assert oracle.normalized_error(np.array([1.0, 0.0, 2.0]), ref, den) == (0.0, 0)
    assert oracle.normalized_error(np.array([1.0, -0.0, 3.0]), ref, den) == (0.25, 2)
    e, i = oracle.normalized_error(np.array([1.0, 1e-30, 2.0]), ref, den)
    assert e == math.inf and i == 1
    e, i = oracle.normalized_error(np.array([np.nan, 0.0, 2.0]), ref, den)
    assert e == math.inf and i == 0


# ------------------------------------------------------------ encoding
# The typed final output rounds the F32 sum to F16 or BF16, nearest with
# ties to even.  oracle.encode is pinned by exhaustive round trips through
# the (separately pinned) decoder, by hand-made ties, and by numpy's and
# torch's own conversions.


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_encode_round_trips_every_16_bit_pattern(dt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.decode(bits, dt)
    keep = ~np.isnan(vals)
    np.testing.assert_array_equal(oracle.encode(vals[keep], dt), bits[keep])


@pytest.mark.parametrize("dt,x,want", [
    ("f16", 1 + 2.0**-11, 0x3C00),          # tie between 1 and 1+2^-10 -> even (1)
    ("f16", 1 + 3 * 2.0**-11, 0x3C02),      # tie between 1+2^-10 and 1+2^-9 -> even
    ("f16", 65520.0, 0x7C00),               # halfway above the largest finite -> inf
    ("f16", 65519.0, 0x7BFF),
    ("f16", 2.0**-25, 0x0000),              # tie between 0 and the smallest subnormal -> 0
    ("f16", 3 * 2.0**-25, 0x0002),          # tie between 1 and 2 subnormal quanta -> 2
    ("f16", -2.0**-14, 0x8400),
    ("bf16", 1 + 2.0**-8, 0x3F80),          # tie -> even (1)
    ("bf16", 1 + 3 * 2.0**-8, 0x3F82),
    ("bf16", -3.0, 0xC040),
])
def test_encode_ties_and_edges(dt, x, want):
    assert int(oracle.encode(np.array([x]), dt)[0]) == want


def test_encode_matches_numpy_and_torch():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000)
    with np.errstate(over="ignore"):
        np.testing.assert_array_equal(oracle.encode(x, "f16"), x.astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(oracle.encode(x, "f32"), x.astype(np.float32).view(np.uint32))
    x32 = x.astype(np.float32).astype(np.float64)  # torch rounds via F32; compare where that is exact
    want = torch.from_numpy(x32).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.encode(x32, "bf16"), want)


def test_truncating_encoder_is_caught():
    """A plausible mistake (truncation instead of rounding) fails the tie pins."""
    x = np.array([1 + 3 * 2.0**-11])
    truncated = (x.astype(np.float32).view(np.uint32) >> 13).astype(np.uint16) - (0x1C000 >> 13)
    assert int(truncated[0]) != int(oracle.encode(x, "f16")[0])
