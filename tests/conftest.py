import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU Monte-Carlo checks")


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_present():
        return
    skip = pytest.mark.skip(reason="no GPU in this container")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per parity check that ran: the coordinates compared with the
    oracle and how many signs differ inside the 1e-5 band (where either
    value is correct; outside it any difference fails the test)."""
    try:
        from gpu_helpers import INBAND_REPORT
    except Exception:
        return
    if not INBAND_REPORT:
        return
    tr = terminalreporter
    tr.section("in-band sign differences (|y| < 1e-5 ||k|| sqrt(d); counted, not failed)")
    for name, coords, inband in INBAND_REPORT:
        frac = inband / coords if coords else 0.0
        tr.write_line(f"{name}: {inband} of {coords} coordinates ({frac:.2e})")
