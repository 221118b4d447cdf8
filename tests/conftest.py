import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C ABI")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    """GPU tests skip (loudly) when no GPU is visible, instead of failing import."""
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Parity margins of the full-size workloads, printed after the test summary
# so that they appear at the end of the run's output even when pytest
# captures each test's own output.
_MARGINS = []


@pytest.fixture
def margin():
    """margin(line): record one line for the end-of-run margin summary."""
    def add(line: str):
        _MARGINS.append(line)
        print(line, flush=True)
    return add


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if _MARGINS:
        terminalreporter.write_sep("-", "parity margins (full-size workloads)")
        for line in _MARGINS:
            terminalreporter.write_line(line)
