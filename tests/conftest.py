import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Max-relative errors of the full-size workload parity cases, printed at the
# end of the run (so they show in `pytest -q` output as well).
_MARGINS = {}


@pytest.fixture
def record_margin():
    def rec(name, rel, tol=2e-3):
        _MARGINS[name] = (rel, tol)
    return rec


def pytest_terminal_summary(terminalreporter):
    if not _MARGINS:
        return
    terminalreporter.write_sep("-", "max|y - y_ref| / max|y_ref| at the workload shapes")
    for name, (rel, tol) in sorted(_MARGINS.items()):
        terminalreporter.write_line(f"{name:48s} {rel:.3e}  ({rel / tol:.0%} of {tol:.0e})")
