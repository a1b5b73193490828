"""bench.py's command-line contract that needs no GPU: asked for more than one
GPU it prints why on stderr, writes no JSON line and exits with status 2,
before it imports torch or touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
