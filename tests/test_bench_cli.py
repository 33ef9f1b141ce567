"""bench.py refuses what it does not measure before it touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_gated_mode_is_forward_only():
    r = _run("--workload", "window", "--mode", "gated", "--pass", "bwd")
    assert r.returncode == 2 and "forward" in r.stderr


def test_gated_mode_is_for_single_calls():
    r = _run("--mode", "gated")
    assert r.returncode == 2 and "single-call" in r.stderr
