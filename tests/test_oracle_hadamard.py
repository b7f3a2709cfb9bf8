"""Pins of the oracle's 128-point Hadamard pre-transform.

ScaleSearch summary page, ScaleSearchAttention, 非干渉処理（IP）と絶対値低減: a
Hadamard transform (as in QuIP#) on Q and K before coding. Reading: the
normalized Sylvester Walsh-Hadamard matrix H/sqrt(128) per 128-vector.
"""
import numpy as np
import scipy.linalg

import workloads


def test_closed_forms(orc):
    x = np.zeros((3, 128), np.float32)
    x[0, :] = 1.0                      # all ones -> sqrt(128) * e0
    x[1, 5] = 1.0                      # one-hot -> row 5 of H / sqrt(128)
    x[2, 0] = -2.0
    y = orc.hadamard128(x)
    assert y[0, 0] == np.float32(np.sqrt(128.0))
    assert np.all(y[0, 1:] == 0)
    c = np.float32(2.0 ** -3.5)
    assert np.all(np.abs(y[1]) == c)
    H = scipy.linalg.hadamard(128)
    np.testing.assert_array_equal(np.sign(y[1]), H[5])
    np.testing.assert_array_equal(y[2], np.float32(-2.0) * c * np.ones(128, np.float32))


def test_matches_library_hadamard(orc):
    x = workloads.workload(5, (1, 2, 64, 128))
    xf = workloads.bf16_bits_to_f32(x).reshape(-1, 128).astype(np.float64)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    ref = ((xf @ H) * np.sqrt(1.0 / 128.0)).astype(np.float32)
    y = orc.hadamard128(x).reshape(-1, 128)
    np.testing.assert_array_equal(y, ref)


def test_involution_and_norm(orc):
    x = workloads.workload(5, (1, 1, 32, 128))
    xf = workloads.bf16_bits_to_f32(x).reshape(-1, 128)
    y = orc.hadamard128(x).reshape(-1, 128)
    z = orc.hadamard128(y).reshape(-1, 128)
    np.testing.assert_allclose(z, xf, rtol=0, atol=2e-6 * np.abs(xf).max())
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-6)


def test_hadamard_then_quantize(orc):
    x = workloads.workload(5, (1, 2, 64, 128))
    y = orc.hadamard128(x)
    c, s, g = orc.quantize(x, -8, 8, hadamard=True)
    c2, s2, g2 = orc.quantize(y.reshape(-1, 128), -8, 8)
    assert g == g2
    np.testing.assert_array_equal(c.reshape(c2.shape), c2)
    np.testing.assert_array_equal(s.reshape(s2.shape), s2)


# --- randomized Hadamard (QuIP#-style random sign flips before the transform) ---

def _signs(seed):
    return np.random.default_rng(seed).integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)


def test_rht_all_positive_signs_is_plain(orc):
    x = workloads.workload(5, (1, 1, 16, 128))
    np.testing.assert_array_equal(orc.hadamard128_rht(x, np.zeros(4, np.uint32)),
                                  orc.hadamard128(x))


def test_rht_matches_library_hadamard_with_signs(orc):
    x = workloads.workload(5, (1, 2, 32, 128))
    w = _signs(3)
    bits = np.array([(w[k // 32] >> (k % 32)) & 1 for k in range(128)])
    s = np.where(bits == 1, -1.0, 1.0)
    xf = workloads.bf16_bits_to_f32(x).reshape(-1, 128).astype(np.float64)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    ref = (((xf * s) @ H) * np.sqrt(1.0 / 128.0)).astype(np.float32)
    np.testing.assert_array_equal(orc.hadamard128_rht(x, w).reshape(-1, 128), ref)


def test_rht_inverse_and_quantize(orc):
    x = workloads.workload(5, (1, 1, 64, 128))
    w = _signs(4)
    bits = np.array([(w[k // 32] >> (k % 32)) & 1 for k in range(128)])
    y = orc.hadamard128_rht(x, w).reshape(-1, 128).astype(np.float64)
    # inverse: x = (y H / sqrt(128)) o s
    H = scipy.linalg.hadamard(128).astype(np.float64)
    back = (y @ H) * np.sqrt(1.0 / 128.0) * np.where(bits == 1, -1.0, 1.0)
    xf = workloads.bf16_bits_to_f32(x).reshape(-1, 128)
    np.testing.assert_allclose(back, xf, rtol=0, atol=1e-6 * np.abs(xf).max())
    c, s, g = orc.quantize_rht(x, w, -8, 8)
    c2, s2, g2 = orc.quantize(orc.hadamard128_rht(x, w).reshape(-1, 128), -8, 8)
    assert g == g2
    np.testing.assert_array_equal(c.reshape(c2.shape), c2)
    np.testing.assert_array_equal(s.reshape(s2.shape), s2)
