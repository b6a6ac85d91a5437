import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# (workload, worst row-relative error, tolerance) recorded by the full-size parity tests
PARITY_RECORDS = []


@pytest.fixture
def record_parity():
    def record(name, err, tol):
        PARITY_RECORDS.append((name, float(err), float(tol)))
    return record


def pytest_terminal_summary(terminalreporter):
    if PARITY_RECORDS:
        terminalreporter.write_sep("-", "GPU vs fp64 oracle: worst row-relative error per workload")
        for name, err, tol in PARITY_RECORDS:
            terminalreporter.write_line(f"{name}: {err:.3e} (tolerance {tol:.0e})")


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
