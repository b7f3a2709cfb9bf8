"""The arithmetic claim behind the certified search on binary32 blocks, checked on
the CPU with the independent NumPy codecs (no GPU, no oracle): split each value
x at fixed bit positions into h (its top 8 significand bits), m (the next 8) and
l (the last 8). Then for every candidate pattern within 8 steps of the default
one (all normal, the default pattern not saturated, block amax in [2^-40, 2^60])
and its E2M1 values V:

- each part is exact in bf16 (its binary32 pattern has a zero low half);
- the terms part_i * V_i of each chain are multiples of 2^(E-14), 2^(E-22) and
  2^(E-30) (E = exponent of the block amax) whose absolute sum stays below 2^24
  of those units, so every partial sum of a chain, in any order and grouping, is
  a binary32 value: the three dot-product chains S1h, S1m, S1l are exact;
- the elements with V_i != 0 are above amax / 64 (what those bounds rest on);
- the remainder m + l is below 2^-7 of x, which bounds S1m + S1l < 2^-7 S1.

Blocks are drawn to stress it: Gaussian, wide exponent spreads, full 24-bit
significands with every low bit set, elements at the smallest magnitudes that
still code nonzero, and block maxima at the edges of the range.
"""
import numpy as np
import pytest

import ref_numpy as R


def _split(x: np.ndarray):
    b = x.view(np.uint32)
    h = (b & np.uint32(0xFFFF0000)).view(np.float32)
    te = (b & np.uint32(0xFFFFFF00)).view(np.float32)
    m = (te - h).astype(np.float32)
    l = (x - te).astype(np.float32)
    return h, m, l


def _blocks(rng, n: int) -> np.ndarray:
    parts = []
    parts.append(rng.standard_normal((n, 16)))
    parts.append(rng.standard_normal((n, 16)) * 2.0 ** rng.integers(-12, 3, (n, 16)))
    # full significands: every low bit set
    g = np.abs(rng.standard_normal((n, 16))).astype(np.float32)
    g = (g.view(np.uint32) | np.uint32(0x0000FFFF)).view(np.float32).astype(np.float64)
    parts.append(g * np.where(rng.random((n, 16)) < 0.5, -1, 1))
    # elements just above the smallest that can code nonzero (amax / 51 .. amax / 40)
    t = rng.uniform(1 / 51, 1 / 40, (n, 16))
    t[:, 0] = 1.0
    parts.append(t * (1.0 + rng.random((n, 16)) * 2.0 ** -10))
    x = np.concatenate(parts).astype(np.float32)
    # block maxima across the range, edges included
    e = rng.choice(np.array([-40, -39, -20, 0, 7, 30, 59]), x.shape[0])
    return (x * np.float32(2.0) ** e[:, None].astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("seed", [1, 2])
def test_three_part_chains_are_exact(seed):
    rng = np.random.default_rng(seed)
    x = _blocks(rng, 2048)
    ax = np.abs(x)
    amax = ax.max(1)
    # a tensor scale per block, 2^-0.5 .. 2^6 times its own amax / 2688, puts the
    # default patterns over the upper normal range (and a few past 448: saturated)
    sg = (amax.astype(np.float64) / 2688.0 *
          2.0 ** rng.uniform(-0.5, 6, amax.shape)).astype(np.float32)
    t = ((amax / np.float32(6)).astype(np.float32) / sg).astype(np.float32)
    p0 = R.e4m3_nearest(t)
    # the certificate's range: all 17 candidates normal, the default pattern not
    # saturated, amax in [2^-40, 2^60]
    ok = (p0 - 8 >= 8) & (t <= 447) & (amax >= 2.0 ** -40) & (amax <= 2.0 ** 60)
    x, ax, amax, p0, sg = x[ok], ax[ok], amax[ok], p0[ok], sg[ok]
    assert x.shape[0] > 4000
    E = np.floor(np.log2(amax.astype(np.float64)))
    h, m, l = _split(x)
    for part in (h, m, l):
        assert not np.any(part.view(np.uint32) & np.uint32(0xFFFF))  # exact in bf16
    xd, hd, md, ld = (a.astype(np.float64) for a in (x, h, m, l))
    assert np.array_equal(hd + md + ld, xd)
    assert np.all(np.abs(md + ld) <= np.abs(xd) * 2.0 ** -7)
    G = R.e2m1_values()
    for f in range(-8, 9):
        p = p0 + f
        live = p <= 126
        d = (R.e4m3_values()[np.clip(p, 0, 126)].astype(np.float32) * sg).astype(np.float32)
        r = (np.float32(1) / d).astype(np.float32)
        V = G[R.e2m1_nearest((ax * r[:, None]).astype(np.float32))] * np.sign(xd)
        V[~live] = 0.0
        nz = V != 0
        assert np.all(ax.astype(np.float64)[nz] > (amax.astype(np.float64)[:, None] / 64)
                      .repeat(16, 1)[nz])
        for part, low in ((hd, 14), (md, 22), (ld, 30)):
            unit = 2.0 ** (E - low)
            terms = part * V / unit[:, None]
            assert np.array_equal(terms, np.round(terms)), f"offset {f}: off the grid"
            assert np.all(np.abs(terms).sum(1) < 2.0 ** 24), f"offset {f}: over 24 bits"
