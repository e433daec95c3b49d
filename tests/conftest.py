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
