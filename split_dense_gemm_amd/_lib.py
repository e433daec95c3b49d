"""ctypes binding of libsplitk.so (argument marshalling only).

Each function takes torch tensors, checks that they are dense device tensors
of the right dtype, and passes their device pointers, sizes and torch's
current HIP stream to the C ABI declared in include/splitk.h.  Every step of
the computation runs in the library's HIP kernels; nothing here computes.
If the library has not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsplitk.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "splitk.h")

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_STATUS_NAMES = {
    0: "SPLITK_OK", 1: "SPLITK_ERR_NULL", 2: "SPLITK_ERR_DTYPE", 3: "SPLITK_ERR_SHAPE",
    4: "SPLITK_ERR_SPLIT", 5: "SPLITK_ERR_ALIAS", 6: "SPLITK_ERR_ALIGN", 7: "SPLITK_ERR_RANGE",
    8: "SPLITK_ERR_LAUNCH", 9: "SPLITK_ERR_WORKSPACE", 10: "SPLITK_ERR_PLAN", 11: "SPLITK_ERR_SCRATCH",
}

LAYOUT_CODE = {"nk": 0, "kn": 1}

_lib = None


class SplitKError(RuntimeError):
    """A non-zero status from the library (nothing was launched)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def library_built() -> bool:
    return os.path.exists(LIB_PATH)


def load():
    """Loads libsplitk.so once.  torch is imported first so that the library
    binds to the HIP runtime torch already mapped (one runtime per process,
    so torch's stream handles are valid in the library)."""
    global _lib
    if _lib is not None:
        return _lib
    if not library_built():
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m split_dense_gemm_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.splitk_gemm_bt.argtypes = [P, P, P, I64, I64, I64, I64, I64, I, P]
    lib.splitk_gemm_bt.restype = I
    lib.splitk_reduce.argtypes = [P, P, I64, I64, I64, P]
    lib.splitk_reduce.restype = I
    lib.splitk_gemm_bt_reduce.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, P]
    lib.splitk_gemm_bt_reduce.restype = I
    lib.splitk_reduce_typed.argtypes = [P, P, I64, I64, I64, I, P]
    lib.splitk_reduce_typed.restype = I
    lib.splitk_gemm_bt_reduce_typed.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.splitk_gemm_bt_reduce_typed.restype = I
    PI64 = ctypes.POINTER(I64)
    lib.splitk_choose_splits.argtypes = [I64, I64, I64, I, I, PI64, PI64, PI64]
    lib.splitk_choose_splits.restype = I
    lib.splitk_gemm_bt_auto.argtypes = [P, P, P, I64, P, I64, I64, I64, I, I, P]
    lib.splitk_gemm_bt_auto.restype = I
    lib.splitk_gemm_bn.argtypes = [P, P, P, I64, I64, I64, I64, I64, I, P]
    lib.splitk_gemm_bn.restype = I
    lib.splitk_gemm_bn_reduce.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.splitk_gemm_bn_reduce.restype = I
    lib.splitk_describe_bn.argtypes = [I64, I64, I64, I64, I64, I, ctypes.c_char_p, I64]
    lib.splitk_describe_bn.restype = I
    lib.splitk_status_str.argtypes = [I]
    lib.splitk_status_str.restype = ctypes.c_char_p
    lib.splitk_reduce_for_gemm.argtypes = [P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.splitk_reduce_for_gemm.restype = I
    lib.splitk_describe.argtypes = [I64, I64, I64, I64, I64, I, ctypes.c_char_p, I64]
    lib.splitk_describe.restype = I
    lib.splitk_gemm_planned.argtypes = [ctypes.c_char_p, I, P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.splitk_gemm_planned.restype = I
    lib.splitk_describe_planned.argtypes = [ctypes.c_char_p, I, I64, I64, I64, I64, I64, I,
                                            ctypes.c_char_p, I64]
    lib.splitk_describe_planned.restype = I
    lib.splitk_gemm_bt_auto_noalloc.argtypes = [P, P, P, I64, I64, I64, I, I, P]
    lib.splitk_gemm_bt_auto_noalloc.restype = I
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/splitk.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(splitk_\w+)\s*\(", text, flags=re.M)


def _check(status: int):
    if status != 0:
        msg = load().splitk_status_str(status).decode()
        raise SplitKError(status, msg)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _operands(A: torch.Tensor, B: torch.Tensor):
    _dev(A, "A")
    _dev(B, "B")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A must be [M,K] and B [N,K]")
    if A.dtype != B.dtype or A.dtype not in DTYPE_CODE:
        raise ValueError(f"A and B must share one of float32/float16/bfloat16, got {A.dtype}, {B.dtype}")
    if A.shape[1] != B.shape[1]:
        raise ValueError(f"A is {tuple(A.shape)} and B is {tuple(B.shape)}: K differs")
    return A.shape[0], B.shape[0], A.shape[1], DTYPE_CODE[A.dtype]


def _operands_kn(A: torch.Tensor, B: torch.Tensor):
    """A [M,K] and B stored [K,N]."""
    _dev(A, "A")
    _dev(B, "B")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A must be [M,K] and B [K,N]")
    if A.dtype != B.dtype or A.dtype not in DTYPE_CODE:
        raise ValueError(f"A and B must share one of float32/float16/bfloat16, got {A.dtype}, {B.dtype}")
    if A.shape[1] != B.shape[0]:
        raise ValueError(f"A is {tuple(A.shape)} and B is {tuple(B.shape)}: K differs")
    return A.shape[0], B.shape[1], A.shape[1], DTYPE_CODE[A.dtype]


def _f32_out(t: torch.Tensor, name: str, numel: int):
    _dev(t, name)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")


def gemm_bt(A: torch.Tensor, B: torch.Tensor, partials: torch.Tensor, k_per_split: int, splits: int,
            stream=None) -> torch.Tensor:
    """partials[s,i,j] = sum over split s's k range of A[i,k]*B[j,k] (see splitk.h)."""
    M, N, K, dt = _operands(A, B)
    _f32_out(partials, "partials", splits * M * N)
    _check(load().splitk_gemm_bt(A.data_ptr(), B.data_ptr(), partials.data_ptr(), M, N, K,
                                 int(k_per_split), int(splits), dt, _stream(stream)))
    return partials


def _out(t: torch.Tensor, numel: int) -> int:
    _dev(t, "C")
    if t.dtype not in DTYPE_CODE:
        raise ValueError(f"C must be float32, float16 or bfloat16, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"C must hold {numel} elements, got {t.numel()}")
    return DTYPE_CODE[t.dtype]


def reduce(partials: torch.Tensor, C: torch.Tensor, splits: int, stream=None) -> torch.Tensor:
    """C[i,j] = sum over s of partials[s,i,j] (see splitk.h).  A float16 or
    bfloat16 C receives the F32 sum rounded to nearest, ties to even."""
    if C.dim() != 2:
        raise ValueError("C must be [M,N]")
    M, N = C.shape
    out = _out(C, M * N)
    _f32_out(partials, "partials", splits * M * N)
    if out == 0:
        _check(load().splitk_reduce(partials.data_ptr(), C.data_ptr(), int(splits), M, N,
                                    _stream(stream)))
    else:
        _check(load().splitk_reduce_typed(partials.data_ptr(), C.data_ptr(), int(splits), M, N, out,
                                          _stream(stream)))
    return C


def reduce_for_gemm(partials: torch.Tensor, C: torch.Tensor, K: int, k_per_split: int, splits: int,
                    dtype, stream=None) -> torch.Tensor:
    """The slab sum of reduce(), for slabs a GEMM of this geometry (K,
    k_per_split, splits, input dtype) has written: the same result bit for
    bit, visiting the plane in that GEMM's tile order (see splitk.h)."""
    if C.dim() != 2:
        raise ValueError("C must be [M,N]")
    M, N = C.shape
    out = _out(C, M * N)
    _f32_out(partials, "partials", splits * M * N)
    _check(load().splitk_reduce_for_gemm(partials.data_ptr(), C.data_ptr(), M, N, int(K),
                                         int(k_per_split), int(splits), _code(dtype), out,
                                         _stream(stream)))
    return C


def gemm_bt_reduce(A: torch.Tensor, B: torch.Tensor, partials: torch.Tensor, C: torch.Tensor,
                   k_per_split: int, splits: int, stream=None) -> torch.Tensor:
    """The split-K GEMM and the slab sum back to back on one stream (see
    splitk.h); C may be float32, float16 or bfloat16."""
    M, N, K, dt = _operands(A, B)
    _f32_out(partials, "partials", splits * M * N)
    out = _out(C, M * N)
    if out == 0:
        _check(load().splitk_gemm_bt_reduce(A.data_ptr(), B.data_ptr(), partials.data_ptr(),
                                            C.data_ptr(), M, N, K, int(k_per_split), int(splits), dt,
                                            _stream(stream)))
    else:
        _check(load().splitk_gemm_bt_reduce_typed(A.data_ptr(), B.data_ptr(), partials.data_ptr(),
                                                  C.data_ptr(), M, N, K, int(k_per_split), int(splits),
                                                  dt, out, _stream(stream)))
    return C


def _code(dtype) -> int:
    return DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)


def choose_splits(M: int, N: int, K: int, dtype, out_dtype=torch.float32):
    """(k_per_split, splits, workspace_elems) the library picks for C = A*B^T
    with an `out_dtype` C (see splitk.h); nothing is launched."""
    kps, s, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().splitk_choose_splits(M, N, K, _code(dtype), _code(out_dtype), ctypes.byref(kps),
                                       ctypes.byref(s), ctypes.byref(ws)))
    return kps.value, s.value, ws.value


def gemm_bt_auto(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, workspace=None,
                 stream=None) -> torch.Tensor:
    """C = A * B^T with the split count the library chooses (see splitk.h).
    `workspace` is a float32 device tensor of at least the elements
    choose_splits() reports, or None when it reports none."""
    M, N, K, dt = _operands(A, B)
    out = _out(C, M * N)
    if workspace is None:
        wp, wn = None, 0
    else:
        _dev(workspace, "workspace")
        if workspace.dtype != torch.float32:
            raise ValueError("workspace must be float32")
        wp, wn = workspace.data_ptr(), workspace.numel()
    _check(load().splitk_gemm_bt_auto(A.data_ptr(), B.data_ptr(), wp, wn, C.data_ptr(), M, N, K, dt,
                                      out, _stream(stream)))
    return C


def gemm_bt_auto_noalloc(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, stream=None) -> torch.Tensor:
    """gemm_bt_auto with the slabs in the library's own static device array
    instead of a workspace (see splitk_gemm_bt_auto_noalloc in splitk.h)."""
    M, N, K, dt = _operands(A, B)
    out = _out(C, M * N)
    _check(load().splitk_gemm_bt_auto_noalloc(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K, dt, out,
                                              _stream(stream)))
    return C


def gemm_bn(A: torch.Tensor, B: torch.Tensor, partials: torch.Tensor, k_per_split: int, splits: int,
            stream=None) -> torch.Tensor:
    """partials[s,i,j] = sum over split s's k range of A[i,k]*B[k,j], with B
    stored [K,N] (see splitk.h)."""
    M, N, K, dt = _operands_kn(A, B)
    _f32_out(partials, "partials", splits * M * N)
    _check(load().splitk_gemm_bn(A.data_ptr(), B.data_ptr(), partials.data_ptr(), M, N, K,
                                 int(k_per_split), int(splits), dt, _stream(stream)))
    return partials


def gemm_bn_reduce(A: torch.Tensor, B: torch.Tensor, partials: torch.Tensor, C: torch.Tensor,
                   k_per_split: int, splits: int, stream=None) -> torch.Tensor:
    """gemm_bn then the slab sum into C (float32, float16 or bfloat16)."""
    M, N, K, dt = _operands_kn(A, B)
    _f32_out(partials, "partials", splits * M * N)
    out = _out(C, M * N)
    _check(load().splitk_gemm_bn_reduce(A.data_ptr(), B.data_ptr(), partials.data_ptr(), C.data_ptr(),
                                        M, N, K, int(k_per_split), int(splits), dt, out,
                                        _stream(stream)))
    return C


def describe_bn(M: int, N: int, K: int, k_per_split: int, splits: int, dtype) -> str:
    """The kernel configuration gemm_bn picks for this problem."""
    buf = ctypes.create_string_buffer(128)
    _check(load().splitk_describe_bn(M, N, K, k_per_split, splits, _code(dtype), buf, len(buf)))
    return buf.value.decode()


def describe(M: int, N: int, K: int, k_per_split: int, splits: int, dtype) -> str:
    """The GEMM kernel configuration the library picks for this problem."""
    code = _code(dtype)
    buf = ctypes.create_string_buffer(128)
    _check(load().splitk_describe(M, N, K, k_per_split, splits, code, buf, len(buf)))
    return buf.value.decode()


def gemm_planned(plan: str, A: torch.Tensor, B: torch.Tensor, partials: torch.Tensor, k_per_split: int,
                 splits: int, C=None, layout: str = "nk", stream=None) -> torch.Tensor:
    """gemm_bt (layout "nk") or gemm_bn (layout "kn") with the kernel
    configuration `plan` names, followed by the slab sum into C when C is
    given (see splitk_gemm_planned in splitk.h).  A test and tuning hook."""
    M, N, K, dt = _operands(A, B) if layout == "nk" else _operands_kn(A, B)
    _f32_out(partials, "partials", splits * M * N)
    out = _out(C, M * N) if C is not None else 0
    _check(load().splitk_gemm_planned(plan.encode(), LAYOUT_CODE[layout], A.data_ptr(), B.data_ptr(),
                                      partials.data_ptr(), None if C is None else C.data_ptr(), M, N, K,
                                      int(k_per_split), int(splits), dt, out, _stream(stream)))
    return partials if C is None else C


def describe_planned(plan: str, M: int, N: int, K: int, k_per_split: int, splits: int, dtype,
                     layout: str = "nk") -> str:
    """The configuration gemm_planned runs for this plan text and problem."""
    buf = ctypes.create_string_buffer(128)
    _check(load().splitk_describe_planned(plan.encode(), LAYOUT_CODE[layout], M, N, K, k_per_split, splits,
                                          _code(dtype), buf, len(buf)))
    return buf.value.decode()


def raw_call(name: str, *args) -> int:
    """Calls a C ABI entry point with raw integer arguments and returns its status
    (used by the tests of the argument checks)."""
    return int(getattr(load(), name)(*args))
