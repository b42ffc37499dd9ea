import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path; tests marked gpu fail loudly if it is not built."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    import rmsnorm_projection_gemm_amd as fn
    fn.load()   # raises if libflashnorm.so is missing
    return fn
