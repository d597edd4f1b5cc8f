import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case (large shapes)")


@pytest.fixture(scope="session")
def sra():
    """The HIP library binding. Fails loudly (never skips) when the library or
    the GPU is missing: a GPU test must not pass on a fallback."""
    import torch  # noqa: F401  (torch's HIP runtime must be loaded first)
    import striped_ring_attention_amd as m
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test collected but no GPU is visible")
    m.load()
    return m
