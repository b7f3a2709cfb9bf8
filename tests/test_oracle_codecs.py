"""Pins of the oracle's two codecs against closed forms and independent nearest searches.

E2M1: 1 sign / 2 exponent / 1 mantissa bit, largest 6 (BEVFormer B200 FP8/FP4
tuning article, 1-A; ScaleSearch summary page, メカニズム: amax / 6.0).
UE4M3: 4 exponent / 3 mantissa bits, largest 448 (same article, 1-A and sec. 7).
"""
import numpy as np
import pytest

import ref_numpy as R


def _floats_between(lo: float, hi: float, stride: int = 1) -> np.ndarray:
    a = np.array([lo], dtype=np.float32).view(np.uint32)[0]
    b = np.array([hi], dtype=np.float32).view(np.uint32)[0]
    return np.arange(a, b + 1, stride, dtype=np.uint32).view(np.float32)


def _window(v: float, n: int) -> np.ndarray:
    u = np.array([v], dtype=np.float32).view(np.uint32)[0].astype(np.int64)
    w = np.arange(max(u - n, 0), u + n + 1, dtype=np.int64).astype(np.uint32)
    return w.view(np.float32)


E2M1_MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def test_e2m1_grid_closed_form(orc):
    # grid from the bit layout: code (e, m), bias 1 -> 0, .5, 1, 1.5, 2, 3, 4, 6
    assert list(R.e2m1_values()) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c, v in enumerate(R.e2m1_values()):
        assert orc.e2m1_code(np.array([v], np.float32))[0] == c


def test_e2m1_midpoints_ties_to_even(orc):
    mids = np.array(E2M1_MIDPOINTS, dtype=np.float32)
    got = orc.e2m1_code(mids)
    # halfway between codes k and k+1 -> the even one of the two
    assert list(got) == [0, 2, 2, 4, 4, 6, 6]
    above = np.nextafter(mids, np.float32(np.inf))
    below = np.nextafter(mids, np.float32(0))
    assert list(orc.e2m1_code(above)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(orc.e2m1_code(below)) == [0, 1, 2, 3, 4, 5, 6]


def test_e2m1_against_nearest_search(orc):
    ys = [_window(m, 1 << 15) for m in E2M1_MIDPOINTS + [6.0]]
    ys.append(_floats_between(0.0, 8.0, stride=997))  # strided sweep of every binade
    ys.append(np.array([0.0, 1e-45, 1.17549435e-38, 6.0, 6.5, 1e30, 3.4e38, np.inf],
                       dtype=np.float32))
    y = np.concatenate(ys)
    np.testing.assert_array_equal(orc.e2m1_code(y), R.e2m1_nearest(y))


def test_e2m1_domain(orc):
    assert orc.e2m1_code(np.array([np.nan, -1.0], np.float32)).tolist() == [-1, -1]


@pytest.mark.slow
def test_e2m1_exhaustive(orc):
    # every non-negative binary32 up to 8.0
    top = int(np.array([8.0], np.float32).view(np.uint32)[0])
    for start in range(0, top + 1, 1 << 24):
        u = np.arange(start, min(start + (1 << 24), top + 1), dtype=np.uint32)
        y = u.view(np.float32)
        np.testing.assert_array_equal(orc.e2m1_code(y), R.e2m1_nearest(y))


def test_e4m3_closed_forms(orc):
    assert orc.e4m3_value(0x33) == 0.6875
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x00) == 0.0
    assert np.isnan(orc.e4m3_value(0x7F))
    vals = np.array([orc.e4m3_value(p) for p in range(127)])
    np.testing.assert_array_equal(vals, R.e4m3_values())
    # strictly increasing: pattern + f is the f-th neighbouring scale
    assert np.all(np.diff(vals) > 0)
    # neighbour ratio inside a normal binade is 1 + 1/(8 + m)
    for p in range(8, 126):
        if (p & 7) != 7:
            assert vals[p + 1] / vals[p] == pytest.approx(1 + 1 / (8 + (p & 7)), rel=0, abs=1e-15)


def test_e4m3_encode_against_nearest_search(orc):
    vals = R.e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    ts = [_window(float(m), 4096) for m in mids]
    ts += [_window(float(v), 64) for v in vals]
    ts.append(_floats_between(0.0, 1024.0, stride=4099))
    ts.append(np.array([0.0, 1e-45, 447.99997, 448.0, 464.0, 480.0, 1e20, np.inf],
                       dtype=np.float32))
    t = np.concatenate(ts)
    np.testing.assert_array_equal(orc.e4m3_encode(t), R.e4m3_nearest(t))


def test_e4m3_encode_ties_and_saturation(orc):
    # 0.65625 is halfway between 0x32 (0.625) and 0x33 (0.6875) -> even pattern 0x32
    assert orc.e4m3_encode(np.array([0.65625], np.float32))[0] == 0x32
    # halfway between 0x33 and 0x34 (0.75) -> 0x34
    assert orc.e4m3_encode(np.array([0.71875], np.float32))[0] == 0x34
    assert orc.e4m3_encode(np.array([448.0, 470.0, 1e30, np.inf], np.float32)).tolist() == [126] * 4
    # half of the smallest subnormal step rounds to zero (tie to the even pattern 0)
    assert orc.e4m3_encode(np.array([2.0 ** -10], np.float32))[0] == 0
    assert orc.e4m3_encode(np.array([np.nan, -1.0], np.float32)).tolist() == [-1, -1]
