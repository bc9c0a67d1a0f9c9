"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a C
driver calls every entry point on ragged sizes (n = 0 .. 4099, groups of
16 .. 1024, per-tensor and per-group activation scales) with exactly-sized
heap buffers and special values; any out-of-bounds access or undefined
behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = os.path.join(tmp_path, "oracle_driver")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", exe, os.path.join(HERE, "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "coat_oracle.c"), "-lm"]
    built = subprocess.run(cmd, capture_output=True, text=True)
    if built.returncode != 0 and "asan" in (built.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not installed: " + built.stderr[-200:])
    assert built.returncode == 0, built.stderr
    # verify_asan_link_order=0: the environment may preload other libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout
