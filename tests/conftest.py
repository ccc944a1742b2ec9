import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size cases (large host-side oracle work)")


def pytest_addoption(parser):
    parser.addoption("--run-benchmark", action="store_true", default=False,
                     help="also run the timing tests")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once; the test fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_tiled_gemm_03_amd as tg
    tg.load()
    return tg
