import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests must never silently pass on a machine without a GPU: they are
    # skipped here only when the run did not ask for them (-m "not gpu").
    pass


@pytest.fixture(scope="session")
def qdg():
    """The HIP library binding; GPU tests fail loudly when it cannot load."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import quantized_dequant_gemm_amd as q
    q.load()  # raises if libqdg.so is missing
    return q
