"""The oracle's search against an independent brute force over all 127 finite scales.

The NumPy reference (tests/ref_numpy.py) scores every block under every E4M3
pattern; restricted to [p0 + f_lo, p0 + f_hi] with the visiting order f = 0,
then f_lo..f_hi, its first strict minimum must be the oracle's choice, with
identical codes. The unrestricted optimum must lie inside a wide range on
Gaussian data (the ScaleSearch summary page, 検索戦略: a small range suffices).
"""
import numpy as np
import pytest

import ref_numpy as R
import workloads


def _as_f32(x):
    return x if x.dtype == np.float32 else workloads.bf16_bits_to_f32(x)


@pytest.mark.parametrize("idx,shape,offs", [
    (1, (16, 1024), (-2, 6)),
    (2, (4, 4096), (-2, 6)),
    (3, (1, 1, 96, 128), (-2, 6)),
    (4, (1, 28672 // 2), (-2, 6)),
    (1, (16, 1024), (-8, 8)),
])
def test_bruteforce_restricted_argmin(orc, idx, shape, offs):
    x = _as_f32(workloads.workload(idx, shape)).reshape(-1, shape[-1])
    c, s, g, f = orc.quantize(x, *offs, want_f=True)
    c2, s2, g2, f2 = R.quantize_ref(x, *offs)
    assert g == g2
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(f, f2)


def test_block_sse_matches_bruteforce_table(orc):
    x = workloads.workload(1, (2, 1024)).reshape(-1, 16)[:20]
    g = np.float32(0.0019)
    table, _ = R.sse_all_patterns(np.abs(x), g)
    for b in range(x.shape[0]):
        for p in range(0, 127, 5):
            assert orc.block_sse(x[b], float(g), p) == table[b, p]


def test_unrestricted_optimum_is_near_default(orc):
    x = workloads.workload(1, (64, 1024))
    _, _, g = orc.quantize(x, -2, 6)
    blocks = np.abs(x.reshape(-1, 16))
    table, _ = R.sse_all_patterns(blocks, g)
    t = ((blocks.max(axis=1) / np.float32(6)).astype(np.float32) / g).astype(np.float32)
    p0 = R.e4m3_nearest(t)
    best = table.argmin(axis=1)
    assert np.all((best - p0 >= -2) & (best - p0 <= 7))


def test_special_values_bruteforce(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    x[0, :16] = 0.0                                  # zero block
    x[1, :16] = np.float32(1e-40)                    # subnormal block
    x[2, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2, np.float32)
    x[3, :] = -x[3, :]
    x[4, 3] = 1000.0                                 # outlier sets the tensor scale
    x[5, :16] = np.float32(5.0)                      # constant block
    x[6, 16:32] = -0.0
    c, s, g, f = orc.quantize(x, -2, 6, want_f=True)
    c2, s2, g2, f2 = R.quantize_ref(x, -2, 6)
    assert g == g2
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(c, c2)
