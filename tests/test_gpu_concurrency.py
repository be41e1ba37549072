"""GPU: the library's calls are thread-safe and stream-independent.  A fresh process
(tests/concurrent_first_calls.py) makes the first calls of several kernel variants from eight
host threads at once, each on its own stream, and compares every thread's results with a
sequential call made afterwards."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_concurrent_first_calls_fresh_process():
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "concurrent_first_calls.py")
    print("[case] concurrent first calls (fresh process)", flush=True)
    r = subprocess.run([sys.executable, script], capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
