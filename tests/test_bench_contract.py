"""bench.py's command-line contract on a machine without a GPU.

More than one GPU is refused with a message (the library has no multi-GPU path), and without a
device the benchmark exits with an error instead of printing a result line: nothing in it falls
back to the CPU.
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    out = _run("--gpus", "2")
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_no_result_line_without_a_gpu():
    if torch.cuda.device_count() > 0:  # counting devices does not initialise one
        pytest.skip("checks the behaviour without a GPU")
    out = _run("--no-secondary", "--steps", "2", "--warmup", "1", "--cpu-seconds", "0.1")
    assert out.returncode != 0
    assert "needs a GPU" in out.stderr
    assert out.stdout.strip() == "", "no JSON line may be printed without a device"
