"""bench.py's command-line contract that needs no GPU: more than one GPU is refused
with a message (this path runs on one GPU), and the options parse."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_measurement_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--config", "--graphs", "--no-granularity",
                 "--no-edges", "--no-dense", "--no-rebuild", "--warm", "--copy-mib"):
        assert flag in r.stdout, flag
