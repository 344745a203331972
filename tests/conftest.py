import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the oracle and the library once if nothing is built yet."""
    from oracle import oracle
    oracle.build_oracle(force=False)


_ensure_built()


@pytest.fixture(scope="session")
def gpu():
    """The torch device for GPU tests; fails loudly when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")
