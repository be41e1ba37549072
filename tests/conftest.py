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
