import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Non-comment, non-empty lines of a golden fixture."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def pytest_terminal_summary(terminalreporter):
    """Print the boundary-window accounting the GPU code checks collected
    (test modules append lines to a module-level WINDOW_REPORT list), so the
    counts appear in a plain -q run too."""
    lines = []
    for name, mod in list(sys.modules.items()):
        rep = getattr(mod, "WINDOW_REPORT", None)
        if isinstance(rep, list) and name.endswith("test_parity_gpu"):
            lines += rep
    if lines:
        terminalreporter.write_sep("-", "code parity: mismatches inside the 1e-6 boundary window (none outside)")
        for ln in lines:
            terminalreporter.write_line(ln)
