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
    """The HIP library binding; loading it fails loudly when the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    from recurrent_lm_sequence_amd import based_la

    return based_la


def pytest_sessionstart(session):
    """Build the HIP library in-tree if (and only if) nothing is built yet."""
    lib = os.path.join(ROOT, "recurrent_lm_sequence_amd", "libbasedla.so")
    if not os.path.exists(lib):
        from recurrent_lm_sequence_amd import _build

        _build.build()
