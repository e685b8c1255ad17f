import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Print every 'err_report' property the tests recorded (the gated tests'
    raw max|err|/rms beside the error beyond fp16 output rounding)."""
    lines = []
    for key in ("passed", "failed"):
        for rep in terminalreporter.stats.get(key, []):
            for name, value in getattr(rep, "user_properties", []):
                if name == "err_report":
                    lines.append(f"{rep.nodeid.split('::')[-1]}  {value}")
    if lines:
        terminalreporter.write_sep("-", "error reports")
        for line in lines:
            terminalreporter.write_line(line)
