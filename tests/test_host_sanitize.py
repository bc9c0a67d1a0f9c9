"""The step library's host-side logic (fp8_optimizer_state_amd/csrc/coat_host.h:
argument checks, step constants, multi-tensor plan tables and their chunked
copy into a workspace or the static table array) under AddressSanitizer and
UndefinedBehaviorSanitizer on the CPU. The same header is compiled into the
library; here a C++ driver calls it with exactly-sized heap buffers on the
Llama-2-13B list (363 tensors), ragged lists and a list filling the static
table, and a second run plants an overrun (a descriptor array one short of
the count passed) that the sanitizer must report."""
import os
import shutil
import subprocess

import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    d = tmp_path_factory.mktemp("host")
    exe = os.path.join(d, "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "fp8_optimizer_state_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "sanitize", "host_driver.cc")]
    built = subprocess.run(cmd, capture_output=True, text=True)
    if built.returncode != 0 and "asan" in (built.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not installed: " + built.stderr[-200:])
    assert built.returncode == 0, built.stderr
    sizes = os.path.join(d, "llama13b_sizes.txt")
    with open(sizes, "w") as f:
        f.write("\n".join(str(n) for n in synth.WORKLOADS["llama13b"].sizes))
    return exe, sizes


def _run(args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run(args, capture_output=True, text=True, env=env, timeout=300)


def test_host_logic_clean_under_asan_ubsan(driver):
    exe, sizes = driver
    assert len(open(sizes).read().split()) == 363
    run = _run([exe, sizes])
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert run.stdout.strip().endswith("ok")


def test_planted_overrun_is_reported(driver):
    exe, sizes = driver
    run = _run([exe, sizes, "overrun"])
    assert run.returncode != 0, run.stdout
    assert "heap-buffer-overflow" in run.stderr, run.stderr[-2000:]
    assert "scan_tensors" in run.stderr
