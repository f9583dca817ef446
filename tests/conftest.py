import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print what every parity check recorded (elements, largest ulp
    distance, elements that passed only through the cancellation floor,
    largest relative error); with RN_PARITY_STATS=<path> also write it as
    JSON."""
    try:
        import tolerance
    except Exception:
        return
    if not tolerance.STATS:
        return
    terminalreporter.section("parity statistics")
    for line in tolerance.summary_lines():
        terminalreporter.write_line(line)
    path = os.environ.get("RN_PARITY_STATS")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(tolerance.STATS, f, indent=1, sort_keys=True)
