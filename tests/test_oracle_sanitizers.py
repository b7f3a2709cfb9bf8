"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only),
driven through every entry point by tests/oracle_sanitize_driver.c: no memory error and
no undefined behaviour on the paths the tests use."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-pthread", os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
