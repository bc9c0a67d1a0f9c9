"""bench.py's command-line contract, host side: it measures one GPU only and
says so for --gpus N > 1, and rejects a non-positive step count, before it
touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_steps_must_be_positive():
    r = _run("--steps", "0")
    assert r.returncode == 2 and r.stdout == ""
