"""bench.py's command line, checked without a GPU: the multi-GPU request is
refused with a message before anything touches the device, and the operand
choices are validated."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_operand_values_are_rejected():
    r = run("--operands", "random")
    assert r.returncode == 2 and "invalid choice" in r.stderr


def test_help_lists_the_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--only", "--operands", "--no-cpu-baseline"):
        assert opt in r.stdout
