"""Host logic of bench.py, on the CPU: the algorithmic byte counts the benchmark divides
by, the refusal of more than one GPU, and the reading of the committed counter summaries
(their source hashes and the search kernel's traffic)."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n_elem,in_bytes,want", [
    (1024 * 1024, 4, 4_784_132),              # FP32 1024 x 1024
    (4096 * 4096, 2, 42_991_620),             # bf16 4096 x 4096
    (8192 * 28672, 2, 601_882_628),           # bf16 8192 x 28672, the benchmark tensor
    (32 * 32768 * 128, 2, 343_932_932),       # bf16 Q [1, 32, 32768, 128]
])
def test_quantize_bytes(n_elem, in_bytes, want):
    """Input once, half a byte of code and a sixteenth of a byte of scale per element,
    and the 4-byte tensor scale."""
    assert bench.quantize_bytes(n_elem, in_bytes) == want


def test_dequantize_bytes_mirror_quantize():
    n = 8192 * 28672
    assert bench.dequantize_bytes(n, 2) == bench.quantize_bytes(n, 2)
    assert bench.dequantize_bytes(n, 4) == bench.quantize_bytes(n, 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_profile_summaries_are_present_and_hashed():
    status = bench.profile_status()
    assert set(status) == set(bench.PROFILES)
    assert all(v in ("current", "stale") for v in status.values()), status
    for name in bench.PROFILES:
        h = bench.recorded_hash(os.path.join(ROOT, "profiles", name))
        assert h is not None and len(h) == 16


def test_committed_search_traffic_matches_the_algorithmic_bytes():
    """The counters' HBM bytes per launch of the search kernel (FETCH_SIZE and
    WRITE_SIZE, calibrated by a plain copy) lie within 0.5% of its algorithmic bytes:
    every byte moves once."""
    if bench.profile_status()["quantize_search_bf16_8192x28672.md"] != "current":
        pytest.skip("the search kernel's counter summary predates its sources")
    t = bench.committed_traffic(bench.SEARCH_KERNEL)
    want = bench.quantize_bytes(bench.ROWS * bench.COLS, 2)
    assert t is not None and abs(t - want) <= 0.005 * want, (t, want)
    frac = bench.committed_valu_issue(bench.SEARCH_KERNEL)
    assert frac is not None and 0.5 < frac <= 1.0
