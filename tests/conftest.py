import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture
def override():
    """Set tuning-table overrides (QG_TUNE, QG_DECODE, ...) through the library
    for one test; all are cleared afterwards."""
    import quantized_gemm_qg_amd as qg

    yield qg.set_override
    qg.clear_overrides()
