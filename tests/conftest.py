import functools
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# Build what the tests load before anything touches the GPU: building starts
# compilers, and a process that has initialised the GPU (gpu_available() below
# does, at collection) must not start other programs.
import split_dense_gemm_amd as _sdg  # noqa: E402

if not _sdg.library_built():
    import __graft_entry__  # noqa: E402

    __graft_entry__.build()
import oracle as _oracle  # noqa: E402

_oracle.ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")


def gpu_available() -> bool:
    try:
        import torch
    except ImportError:
        return False
    return bool(torch.cuda.is_available())


@pytest.fixture(scope="session")
def hip_lib():
    """The built HIP library, built first if nothing is there yet."""
    import split_dense_gemm_amd as sdg

    if not sdg.library_built():
        import __graft_entry__

        __graft_entry__.build()
    return sdg


LARGEST = "bf16_m2048_n4096_k4096_s8"


@functools.lru_cache(maxsize=1)
def largest_reference():
    """Operands of the 2048x4096x4096, 8-split BF16 workload and its whole
    binary64 reference, computed once per session and shared by the tests
    that compare every output of that workload: (a, b, RP, DP, RC, DC) with
    RP/DP the [8,M,N] partials and their error scales, RC/DC the unsplit
    product and its scale (about 1.2 GB of host memory)."""
    from split_dense_gemm_amd import inputs

    w = inputs.WORKLOADS[LARGEST]
    a, b = inputs.workload_operands(w)
    a64 = _oracle.decode(inputs.stored_bits(a), w.dtype)
    b64 = _oracle.decode(inputs.stored_bits(b), w.dtype)
    RP, DP, _ = _oracle.splitk_partials(a64, b64, w.kps, w.splits)
    RC, DC, _ = _oracle.gemm_bt(a64, b64)
    return a, b, RP, DP, RC, DC
