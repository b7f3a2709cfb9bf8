"""Pins of the oracle's MXFP4 contrast format.

Pages: "NVIDIAのFP4推論が50倍の効率を実現", 超低精度推論を支えるアーキテクチャ (NVFP4's
E4M3 block scale and FP32 tensor scale against MXFP4's power-of-two scaling);
ScaleSearch summary page, 手法 > ScaleSearch (the offset search, here over E8M0
exponents). Reading of MXFP4 itself (the pages do not define it): the OCP
Microscaling v1.0 format, 32-element blocks, E8M0 scale 2^X with
X = floor(log2 amax) - 2, E2M1 elements nearest-even with saturation.
"""
import numpy as np
import pytest

import ref_numpy
import workloads


def blk(vals, n=32):
    x = np.zeros((1, n), np.float32)
    x[0, :len(vals)] = vals
    return x


def nibbles(codes):
    c = codes.reshape(-1)
    out = np.empty(c.size * 2, np.uint8)
    out[0::2] = c & 0xF
    out[1::2] = c >> 4
    return out


def test_closed_forms(orc):
    # amax 6 = 1.5 * 2^2 -> X = 0 (byte 127); grid values code exactly
    c, s = orc.quantize_mxfp4(blk([6, -3, 1.5, 0.5, -0.0, 4, 2, 1]))
    assert s[0, 0] == 127
    assert list(nibbles(c)[:8]) == [7, 0x8 | 5, 3, 1, 0x8, 6, 4, 2]
    # amax 7 -> floor(log2 7) = 2 -> X = 0: 7 clips to 6 (the OCP rule's known clipping)
    c, s = orc.quantize_mxfp4(blk([7.0]))
    assert s[0, 0] == 127 and nibbles(c)[0] == 7
    # amax 8 -> X = 1 (byte 128): 8 / 2 = 4 -> code 6
    c, s = orc.quantize_mxfp4(blk([8.0, 1.0]))
    assert s[0, 0] == 128 and list(nibbles(c)[:2]) == [6, 1]
    # amax 0.75 = 1.5 * 2^-1 -> X = -3: 0.75 * 8 = 6
    c, s = orc.quantize_mxfp4(blk([0.75]))
    assert s[0, 0] == 124 and nibbles(c)[0] == 7
    # all zero: X = -127 (byte 0), codes keep the input's zero signs
    c, s = orc.quantize_mxfp4(blk([0.0, -0.0]))
    assert s[0, 0] == 0 and list(nibbles(c)[:2]) == [0, 8]
    # non-finite: byte 255, codes 0
    c, s = orc.quantize_mxfp4(blk([1.0, np.inf]))
    assert s[0, 0] == 255 and np.all(c == 0)
    y = orc.dequantize_mxfp4(c, s)
    assert np.all(np.isnan(y))


def test_search_prefers_larger_scale_when_clipping(orc):
    # amax 7 clips to 6 at X = 0 (error 1); at X = 1, 7/2 = 3.5 ties between 3 and 4
    # and takes the even code (4 -> 8): error 1 as well, so f = 0 keeps the tie.
    x = blk([7.0])
    assert orc.mx_block_sse(x, 0) == 1.0 and orc.mx_block_sse(x, 1) == 1.0
    c, s = orc.quantize_mxfp4(x, -1, 1)
    assert s[0, 0] == 127
    # amax 7.5: X = 0 gives error 1.5^2; X = 1 gives 3.75 -> 4 -> 8, error 0.25
    x = blk([7.5])
    c, s = orc.quantize_mxfp4(x, -1, 1)
    assert s[0, 0] == 128 and nibbles(c)[0] == 6
    c, s = orc.quantize_mxfp4(x, 0, 0)
    assert s[0, 0] == 127


def test_matches_bruteforce(orc):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    x[5, 40] = 1e-40  # subnormal in a block
    for lo, hi in [(0, 0), (-1, 1), (-3, 2)]:
        c, s = orc.quantize_mxfp4(x, lo, hi)
        rc, rs = ref_numpy.mx_quantize_ref(x, lo, hi)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(c, rc)


def test_invariants(orc):
    x = workloads.bf16_bits_to_f32(workloads.workload(2, (64, 512)))
    c, s = orc.quantize_mxfp4(x, -1, 1)
    # power-of-two scaling moves the exponent byte only
    for k in (-5, 3):
        ck, sk = orc.quantize_mxfp4((x * np.float32(2.0 ** k)).astype(np.float32), -1, 1)
        np.testing.assert_array_equal(ck, c)
        np.testing.assert_array_equal(sk.astype(int), s.astype(int) + k)
    # sign symmetry
    cn, sn = orc.quantize_mxfp4(-x, -1, 1)
    np.testing.assert_array_equal(cn, c ^ 0x88)
    np.testing.assert_array_equal(sn, s)
    # bf16 input equals its FP32 widening; thread count does not matter
    xb = workloads.workload(2, (64, 512))
    np.testing.assert_array_equal(orc.quantize_mxfp4(xb, -1, 1)[0], c)
    np.testing.assert_array_equal(orc.quantize_mxfp4(x, -1, 1, nthreads=1)[1], s)


def test_round_trip_and_max_scaling_range(orc):
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    v = grid[rng.integers(0, 8, (16, 64))] * np.where(rng.random((16, 64)) < 0.5, -1, 1)
    v[:, ::32] = 6.0  # every block's amax is 6 -> X = 0
    X = rng.integers(-20, 20, (16, 2)).repeat(32, axis=1)
    x = (v * np.exp2(X)).astype(np.float32)
    c, s = orc.quantize_mxfp4(x)
    np.testing.assert_array_equal(orc.dequantize_mxfp4(c, s), x)
    # with [0, 0] every block's amax lands in [4, 8) * 2^X
    y = workloads.bf16_bits_to_f32(workloads.workload(4, (32, 1024)))
    c, s = orc.quantize_mxfp4(y)
    amax = np.abs(y.reshape(-1, 32)).max(axis=1)
    ratio = amax / np.exp2(s.reshape(-1).astype(np.float64) - 127)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_search_never_worse(orc):
    x = workloads.bf16_bits_to_f32(workloads.workload(2, (128, 1024)))
    e = {}
    for r in [(0, 0), (-1, 1)]:
        c, s = orc.quantize_mxfp4(x, *r)
        y = orc.dequantize_mxfp4(c, s)
        e[r] = ((y.astype(np.float64) - x) ** 2).reshape(-1, 32).sum(axis=1)
    assert np.all(e[(-1, 1)] <= e[(0, 0)] * (1 + 1e-6) + 1e-30)
    assert e[(-1, 1)].sum() < e[(0, 0)].sum()


def test_dequantize_bf16(orc):
    x = workloads.bf16_bits_to_f32(workloads.workload(4, (8, 256)))
    c, s = orc.quantize_mxfp4(x, -1, 1)
    yf = orc.dequantize_mxfp4(c, s)
    yb = orc.dequantize_mxfp4(c, s, out="bf16")
    np.testing.assert_array_equal(yb, workloads.to_bf16_bits(yf))
