"""The benchmark's command-line contract that needs no GPU: more than one
GPU is refused with a message and exit status 2."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                            "--gpus", str(n)], capture_output=True, text=True,
                           timeout=120)
        assert p.returncode == 2
        assert f"--gpus {n} is not supported" in p.stderr
        assert "one GPU" in p.stderr
        assert p.stdout == ""
