"""nvfp4_quantize_noalloc (the allocation-free quantize: the amax pass's partial
maxima in a library-owned device array instead of a workspace) gives exactly the
bytes of nvfp4_quantize, the entry point it mirrors, on consecutive calls whose
second input is smaller than the first (the array keeps the last call's
contents), with and without the Hadamard transform and a given tensor scale."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    ha, hb = to_host(a), to_host(b)
    assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), what + ": " + first_mismatch(ha, hb)


def _check(nv, xh, offsets, hadamard=False, given=False):
    print(f"[case] noalloc {xh.shape} {xh.dtype} offsets={offsets} hadamard={hadamard} "
          f"given={given}", flush=True)
    x = to_dev(xh)
    gs = None
    if given:
        gs = nv.global_scale(x, hadamard=hadamard)
    c1, s1, g1 = nv.quantize(x, offsets, hadamard=hadamard, global_scale=gs)
    c2, s2, g2 = nv.quantize_noalloc(x, offsets, hadamard=hadamard, global_scale=gs)
    torch.cuda.synchronize()
    _same(g2, g1, "tensor scale")
    _same(s2, s1, "scales")
    _same(c2, c1, "codes")


def test_scratch_size(gpu):
    assert gpu.load().nvfp4_noalloc_scratch_bytes() == 2048


@pytest.mark.parametrize("hadamard", [False, True])
def test_noalloc_matches_quantize_large_then_small(gpu, hadamard):
    big = workloads.workload(4, (1024, 28672 // 2))       # 3584 partial-max workgroups' worth
    small = workloads.workload(4, (37, 1024))              # a few workgroups, ragged
    offs = (-8, 8) if hadamard else (-2, 6)
    _check(gpu, big, offs, hadamard)
    _check(gpu, small, offs, hadamard)


def test_noalloc_fp32_and_given_scale(gpu):
    x = workloads.workload(1)                              # FP32 1024 x 1024
    _check(gpu, x, (-2, 6))
    _check(gpu, x[:3], (-2, 6), given=True)
    _check(gpu, x[:5, :48], (0, 0))


def test_noalloc_empty_and_nonfinite(gpu):
    x = workloads.workload(1, (8, 64)).copy()
    x[3, 17] = np.inf
    _check(gpu, x, (-2, 6))
    _check(gpu, x[:0], (-2, 6))
