"""ctypes wrapper around oracle.c, the binary64 split-K reference.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and bench.py's CPU
baseline leg may import this; the product path never does.

Every function follows the definition on the pages ("Aligned shared rows
for pipelined NAX on CUDA", section "Contract and correctness"; "Wider
consecutive-weight NAX GEMM", section "Launch contract and correctness"):
partials[s,i,j] is the sum over split s's k range of A[i,k]*B[j,k], the final
output is the sum over all k, and every check uses binary64 products of the
stored (already rounded) inputs.  The numeric work happens in oracle.c; this
file only marshals numpy arrays.

Parity pins for each function are in tests/test_oracle.py (IEEE bit
patterns, torch's decoder, exact rational brute force, numpy's float64
GEMM, closed forms, invariants, and mutants that the pins must reject).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

_DTYPE = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build() -> str:
    """Compile oracle.c with the host C compiler (no fast-math)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC,
           "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def ensure_built():
    """Builds (if missing or older than oracle.c) and loads the reference.
    Call it before the process touches the GPU: building starts the host
    compiler, and a process that has initialised the GPU must not start
    other programs."""
    _load()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_decode.argtypes = [P, ctypes.c_int, I64, P]
    lib.oracle_encode.argtypes = [P, ctypes.c_int, I64, P]
    lib.oracle_splitk_partials.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, ctypes.c_int]
    lib.oracle_gemm_bt.argtypes = [P, P, I64, I64, I64, P, P, ctypes.c_int]
    lib.oracle_slab_sum.argtypes = [P, I64, I64, I64, P, P, ctypes.c_int]
    lib.oracle_sampled.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, I64, P, P, P, P]
    lib.oracle_threads.argtypes = [ctypes.c_int, I64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def threads_for(nthreads: int, rows: int) -> int:
    """Worker threads a call with `nthreads` (0 = every online core) uses."""
    return int(_load().oracle_threads(int(nthreads), int(rows)))


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact binary64 values of stored elements (uint16 for F16/BF16, uint32 for F32)."""
    want = np.uint32 if dtype == "f32" else np.uint16
    bits = np.ascontiguousarray(bits)
    if bits.dtype != want:
        raise TypeError(f"{dtype} bits must be {want.__name__}, got {bits.dtype}")
    out = np.empty(bits.shape, dtype=np.float64)
    rc = _load().oracle_decode(_ptr(bits), _DTYPE[dtype], bits.size, _ptr(out))
    if rc != 0:
        raise ValueError(dtype)
    return out


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """Bits of binary64 values rounded to `dtype` (nearest, ties to even).

    Used for typed final outputs: the split-K sum rounded to F16 or BF16.
    """
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=np.uint32 if dtype == "f32" else np.uint16)
    rc = _load().oracle_encode(_ptr(values), _DTYPE[dtype], values.size, _ptr(out))
    if rc != 0:
        raise ValueError(dtype)
    return out


def splitk_partials(a: np.ndarray, b: np.ndarray, kps: int, splits: int, nthreads: int = 0):
    """(P, DP, threads): P[s,i,j] over split s's k range, DP the sum of |terms|."""
    a, b = _f64(a), _f64(b)
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    P = np.empty((splits, M, N), dtype=np.float64)
    DP = np.empty_like(P)
    rc = _load().oracle_splitk_partials(_ptr(a), _ptr(b), M, N, K, kps, splits, _ptr(P), _ptr(DP),
                                        int(nthreads))
    if rc < 0:
        raise ValueError(f"split geometry K={K} kps={kps} splits={splits} is not allowed")
    return P, DP, rc


def gemm_bt(a: np.ndarray, b: np.ndarray, nthreads: int = 0):
    """(C, DC, threads): the unsplit product over all k, computed on its own."""
    a, b = _f64(a), _f64(b)
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    C = np.empty((M, N), dtype=np.float64)
    DC = np.empty_like(C)
    rc = _load().oracle_gemm_bt(_ptr(a), _ptr(b), M, N, K, _ptr(C), _ptr(DC), int(nthreads))
    if rc < 0:
        raise ValueError("bad shape")
    return C, DC, rc


def slab_sum(slabs: np.ndarray, nthreads: int = 0):
    """(C, D, threads): binary64 sum over s of F32 slabs[s,i,j], D the sum of |values|."""
    slabs = np.ascontiguousarray(slabs, dtype=np.float32)
    S, M, N = slabs.shape
    C = np.empty((M, N), dtype=np.float64)
    D = np.empty_like(C)
    rc = _load().oracle_slab_sum(_ptr(slabs), S, M, N, _ptr(C), _ptr(D), int(nthreads))
    if rc < 0:
        raise ValueError("bad shape")
    return C, D, rc


def sampled(a: np.ndarray, b: np.ndarray, kps: int, splits: int, rows, cols):
    """Reference values at chosen (row, col) pairs: (P[t,s], DP[t,s], C[t], DC[t])."""
    a, b = _f64(a), _f64(b)
    M, K = a.shape
    N, _ = b.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = rows.size
    P = np.empty((n, splits), dtype=np.float64)
    DP = np.empty_like(P)
    C = np.empty(n, dtype=np.float64)
    DC = np.empty_like(C)
    rc = _load().oracle_sampled(_ptr(a), _ptr(b), M, N, K, kps, splits, _ptr(rows), _ptr(cols), n,
                                _ptr(P), _ptr(DP), _ptr(C), _ptr(DC))
    if rc != 0:
        raise ValueError(f"oracle_sampled rejected its arguments ({rc})")
    return P, DP, C, DC


def normalized_error(got: np.ndarray, ref: np.ndarray, denom: np.ndarray):
    """Largest |got - ref| / denom and its flat index.

    The pages state tolerances but not the error measure; the measure used
    here divides by the sum of |products| that make up the reference value.
    Where that sum is zero the result must be exactly zero (either sign), and
    anything else, NaN included, counts as an infinite error.
    """
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    denom = np.asarray(denom, dtype=np.float64).ravel()
    if got.shape != ref.shape or ref.shape != denom.shape:
        raise ValueError("shape mismatch")
    if got.size == 0:
        return 0.0, -1
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(denom > 0, diff / np.where(denom > 0, denom, 1.0),
                       np.where(got == 0, 0.0, np.inf))
    err = np.where(np.isnan(err), np.inf, err)
    idx = int(np.argmax(err))
    return float(err[idx]), idx
