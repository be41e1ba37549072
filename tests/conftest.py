"""Shared pytest configuration.

Markers:
  gpu  -- needs an MI355X (gfx950) device and the built HIP library.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: test needs an AMD GPU (gfx950) and the built library")
    config.fullsize_lines = []   # per-workload results of the full-size GPU parity test


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the full-size parity results (whole-tensor mismatch fractions, boundary cases, worst
    rotation error) after the run, where a quiet run still shows them."""
    lines = getattr(config, "fullsize_lines", [])
    if lines:
        terminalreporter.write_line("full-size parity, every row of each workload:")
        for line in lines:
            terminalreporter.write_line("  " + line)
