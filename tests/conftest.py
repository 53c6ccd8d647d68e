"""Shared pytest setup: the ``gpu`` marker, the repository root on sys.path, and the
end-of-session table of GPU parity margins."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    import parity_log

    lines = parity_log.summary_lines()
    if not lines:
        return
    terminalreporter.section("parity margins against the fp64 oracle")
    for line in lines:
        terminalreporter.write_line(line)
