"""The host side of the C-ABI library under AddressSanitizer and UndefinedBehavior-
Sanitizer: the library's sources are built again with the sanitizers on the host
compilation only (the gfx950 device code is unchanged), then tests/test_abi.py (every
exported symbol; every argument check, which runs before any launch) is run against
that copy in a child process with the ASan runtime preloaded. No GPU is used."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    from microscaling_fp4_block_amd import build

    out = str(tmp_path / "libnvfp4_asan.so")
    host_only = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        host_only += ["-Xarch_host", flag]
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + host_only
    cmd = [build.hipcc()] + flags + [os.path.join(build.CSRC, s) for s in build.SOURCES] + ["-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, NVFP4_ABI_TEST_LIB=out, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True,
                       env=env, cwd=ROOT, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
