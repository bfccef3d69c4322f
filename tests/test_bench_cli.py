"""The benchmark's command-line contract that needs no GPU: it measures one
GPU only and refuses more with a message and a non-zero status."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""      # no JSON line
