"""Host-side thread safety (needs an MI355X): in a fresh process four threads
make their first library calls at the same time (per-device kernel set-up,
planning, table copies and launches on four streams, both precisions), and
every result equals the same step run alone."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_concurrent_first_calls_from_four_threads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "gpu_threads_child.py")], capture_output=True,
                       text=True, timeout=240, cwd=ROOT)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("same")
