"""bench.py command line, on the CPU: the one-GPU refusal and the no-GPU path
(no projection runs here)."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_no_gpu_fails_loudly():
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu", "--warm-seconds", "0")
    assert r.returncode == 1
    assert json.loads(r.stdout.strip().splitlines()[-1]) == {"error": "no GPU visible"}


def test_help_lists_the_warm_up_options():
    r = _run("--help")
    assert r.returncode == 0
    assert "--warmup" in r.stdout and "--warm-seconds" in r.stdout
