"""Split-K dense GEMM for AMD MI355X (gfx950).

C[M,N] = A[M,K] . B[N,K]^T, computed as F32 partial slabs per K split by a
hand-written CDNA4 MFMA kernel and summed into C by a separate slab-reduce
kernel.  The C ABI is include/splitk.h; this package is a thin ctypes binding
over it (torch provides device memory and streams only).
"""
from ._lib import (  # noqa: F401
    DTYPE_CODE,
    SplitKError,
    choose_splits,
    describe,
    describe_bn,
    describe_planned,
    gemm_bn,
    gemm_bn_reduce,
    gemm_bt,
    gemm_bt_auto,
    gemm_bt_auto_noalloc,
    gemm_bt_reduce,
    gemm_planned,
    header_functions,
    library_built,
    load,
    raw_call,
    reduce,
    reduce_for_gemm,
)
