"""F64 CPU reference for split-K GEMM and the slab sum.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of bench.py.  The product library never imports or links it.
"""
from .ref import (  # noqa: F401
    build,
    decode,
    encode,
    ensure_built,
    gemm_bt,
    normalized_error,
    sampled,
    slab_sum,
    splitk_partials,
    threads_for,
)
