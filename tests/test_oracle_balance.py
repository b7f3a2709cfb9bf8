"""Pins of the oracle's balancing pair (ScaleSearch summary page, ScaleSearchAttention,
非干渉処理（IP）と絶対値低減: an additional pair Q' = Q R^-T, K' = K R that keeps the
attention scores and lowers the mean-square magnitude of the projected tensors).

Reading (the pages fix neither R nor how it is found): R = diag(2^e) over the
channels, e_j the integer in [-16, 16] that minimises channel j's share
a^2 4^-e + b^2 4^e of ||Q'||^2 + ||K'||^2 (a^2, b^2 the channel's sums of squares
in Q and K; ties to the smaller e; 0 when either is 0); with the Hadamard
transform the pair acts first."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import workloads


def brute_exponent(a2: float, b2: float) -> int:
    """Exact argmin over e in [-16, 16] of a2 4^-e + b2 4^e (rationals), least e on a tie."""
    if not (a2 > 0 and b2 > 0):
        return 0
    A, Bq = Fraction(a2), Fraction(b2)
    costs = [(A / Fraction(4) ** e + Bq * Fraction(4) ** e, e) for e in range(-16, 17)]
    best = min(c for c, _ in costs)
    return min(e for c, e in costs if c == best)


def test_exponent_rule_against_exact_brute_force(orc):
    rng = np.random.default_rng(0)
    cases = [(1.0, 1.0), (64.0, 0.25), (16.0, 1.0), (4.0, 1.0), (4.0 * (1 + 2**-52), 1.0),
             (1.0, 4.0), (0.0, 3.0), (3.0, 0.0), (0.0, 0.0), (1e300, 1e-300), (1e-300, 1e300),
             (2.0 ** 40, 1.0), (1.0, 2.0 ** -70)]
    # exact ties: a2 = b2 4^(2e+1) (f(e) = f(e+1)), and one ulp to either side
    for e in range(-4, 5):
        t = 4.0 ** (2 * e + 1)
        cases += [(t, 1.0), (np.nextafter(t, 0), 1.0), (np.nextafter(t, np.inf), 1.0)]
    cases += [tuple(float(v) for v in rng.lognormal(0, 4, 2)) for _ in range(300)]
    for a2, b2 in cases:
        assert orc.balance_exponent(a2, b2) == brute_exponent(a2, b2), (a2, b2)


def test_two_channel_closed_form(orc):
    """Q channel 0 at 8, K channel 0 at 0.5: a^2 / b^2 = 256, so e = 2 and both become
    2 (f(2) = 8 N against f(1) = f(3) = 17 N); channel 1 equal in Q and K keeps e = 0."""
    N = 64
    q = np.zeros((N, 16), np.float32)
    k = np.zeros((N, 16), np.float32)
    q[:, 0], k[:, 0] = 8.0, 0.5
    q[:, 1], k[:, 1] = 3.0, -3.0
    e = orc.balance_exponents(q, k)
    assert e[0] == 2 and e[1] == 0 and np.all(e[2:] == 0)
    np.testing.assert_array_equal(np.ldexp(q[:, 0], -e[0]), np.full(N, 2.0))
    np.testing.assert_array_equal(np.ldexp(k[:, 0], e[0]), np.full(N, 2.0))


def kq(D=128, n=512, seed=0):
    """K of the KV workload recipe (per-channel log-normal scales) and N(0, 1) Q, bf16."""
    k = workloads.workload(3, (1, 1, n, D))
    q = workloads.to_bf16_bits(np.random.default_rng(seed).standard_normal((1, 1, n, D))
                               .astype(np.float32))
    return q, k


def test_calibration_matches_column_sums(orc):
    """Exponents from the oracle's double column sums against NumPy's (exact here: bf16
    squares summed in double) and the exact rule."""
    q, k = kq()
    Q, K = workloads.bf16_bits_to_f32(q).reshape(-1, 128), workloads.bf16_bits_to_f32(k).reshape(-1, 128)
    a2 = (Q.astype(np.float64) ** 2).sum(0)
    b2 = (K.astype(np.float64) ** 2).sum(0)
    e = orc.balance_exponents(q, k)
    assert [int(v) for v in e] == [brute_exponent(x, y) for x, y in zip(a2, b2)]
    assert np.any(e != 0)


def test_scores_kept_and_energy_lowered(orc):
    """QK^T is kept exactly (power-of-two channel factors); ||Q'||^2 + ||K'||^2 does not
    exceed ||Q||^2 + ||K||^2, falls strictly here, and is unchanged for balanced data."""
    q, k = kq()
    Q = workloads.bf16_bits_to_f32(q).reshape(-1, 128).astype(np.float64)
    K = workloads.bf16_bits_to_f32(k).reshape(-1, 128).astype(np.float64)
    e = orc.balance_exponents(q, k).astype(np.int64)
    Qp, Kp = np.ldexp(Q, -e), np.ldexp(K, e)
    np.testing.assert_array_equal(Qp @ Kp.T, Q @ K.T)
    before = (Q ** 2).sum() + (K ** 2).sum()
    after = (Qp ** 2).sum() + (Kp ** 2).sum()
    assert after < 0.95 * before
    # per channel never above the identity's share
    assert np.all((Qp ** 2).sum(0) + (Kp ** 2).sum(0) <= (Q ** 2).sum(0) + (K ** 2).sum(0))
    # already balanced: K = Q gives e = 0 everywhere
    assert np.all(orc.balance_exponents(q, q) == 0)


def test_quantize_is_the_quantizer_of_the_scaled_tensor(orc):
    """Without the transform, one side of the pair is the quantizer of the binary32
    tensor x 2^(side e); with e = 0 it is the plain quantizer."""
    q, k = kq(n=96)
    e = orc.balance_exponents(q, k)
    for x, side in ((q, -1), (k, 1)):
        xs = np.ldexp(workloads.bf16_bits_to_f32(x), side * e.astype(np.int64)).astype(np.float32)
        got = orc.quantize_balanced(x, e, side, -2, 6)
        ref = orc.quantize(xs, -2, 6)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)
    zero = np.zeros(128, np.int8)
    for a, b in zip(orc.quantize_balanced(k, zero, 1, -2, 6), orc.quantize(k, -2, 6)):
        np.testing.assert_array_equal(np.asarray(a).reshape(-1), np.asarray(b).reshape(-1))


def test_hadamard_after_the_pair(orc):
    """With the transform: y = (x 2^(side e) o s) H / sqrt(128), against scipy's Hadamard
    matrix in double (within one rounding to binary32); scores kept to FP32 rounding;
    e = 0 gives the randomized transform bit for bit."""
    q, k = kq(n=64)
    e = orc.balance_exponents(q, k)
    signs = np.random.default_rng(3).integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)
    bits = ((signs[np.arange(128) // 32] >> (np.arange(128) % 32)) & 1).astype(np.float64)
    s = 1.0 - 2.0 * bits
    H = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128.0)
    ys = {}
    for x, side in ((q, -1), (k, 1)):
        X = workloads.bf16_bits_to_f32(x).reshape(-1, 128).astype(np.float64)
        ref = (np.ldexp(X, side * e.astype(np.int64)) * s) @ H
        y = orc.hadamard128_balanced(x.reshape(-1, 128), e, side, signs).astype(np.float64)
        np.testing.assert_allclose(y, ref, rtol=2.0 ** -23, atol=1e-30)
        ys[side] = y
    Q = workloads.bf16_bits_to_f32(q).reshape(-1, 128).astype(np.float64)
    K = workloads.bf16_bits_to_f32(k).reshape(-1, 128).astype(np.float64)
    S = Q @ K.T
    mag = np.abs(Q) @ np.abs(K).T
    assert np.all(np.abs(ys[-1] @ ys[1].T - S) <= 1e-6 * mag)
    zero = np.zeros(128, np.int8)
    np.testing.assert_array_equal(orc.hadamard128_balanced(k.reshape(-1, 128), zero, 1, signs),
                                  orc.hadamard128_rht(k.reshape(-1, 128), signs))
    # the fused quantize equals the quantizer of the transform
    c, sc, g = orc.quantize_balanced(k, e, 1, -8, 8, hadamard=True, signs=signs)
    rc, rs, rg = orc.quantize(ys[1].astype(np.float32), -8, 8)
    np.testing.assert_array_equal(c.reshape(rc.shape), rc)
    np.testing.assert_array_equal(sc.reshape(rs.shape), rs)
    assert g == rg


def test_exponents_clamped_and_bad_arguments(orc):
    """Exponents beyond [-32, 32] act as +-32; a side other than +-1 or a wrong-length
    exponent array is rejected."""
    x = workloads.to_bf16_bits(np.random.default_rng(4).standard_normal((4, 128)).astype(np.float32))
    for a, b in zip(orc.quantize_balanced(x, np.full(128, 100, np.int8), 1),
                    orc.quantize_balanced(x, np.full(128, 32, np.int8), 1)):
        np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        orc.quantize_balanced(x, np.zeros(128, np.int8), 2)
    with pytest.raises(ValueError):
        orc.quantize_balanced(x, np.zeros(64, np.int8), 1)
