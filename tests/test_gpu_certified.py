"""The certified search (bf16 values with exact one-part sums; binary32 values,
the Hadamard path's among them, with exact three-part sums) must give the
contract's result on blocks where the certificate cannot decide: candidates whose
SSEs tie exactly or differ by a few parts per million, and twins eight patterns
apart whose codes reconstruct every element alike. Inputs are chosen on the CPU
with the independent NumPy reference (no GPU output is used to build them);
results are compared bit for bit with the oracle under the same tensor scale."""
import numpy as np
import pytest
import torch

import ref_numpy as R
import workloads
from gpu_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def _relative_gaps(blocks_f32, sg, lo, hi):
    ax = np.abs(blocks_f32)
    t = ((ax.max(1) / np.float32(6)).astype(np.float32) / np.float32(sg)).astype(np.float32)
    p0 = R.e4m3_nearest(t)
    sse = []
    for f in range(lo, hi + 1):
        p = p0 + f
        s, _ = R.sse_patterns(ax, np.float32(sg), np.clip(p, 0, 126))
        sse.append(np.where((p >= 0) & (p <= 126), s, np.inf))
    sse = np.sort(np.stack(sse, 1).astype(np.float64), axis=1)
    return (sse[:, 1] - sse[:, 0]) / np.maximum(sse[:, 0], 1e-300)


def check_given(nv, orc, xh, sg, offsets):
    print(f"[case] {xh.shape} offsets={offsets} S_g={sg!r}", flush=True)
    g = torch.tensor([sg], dtype=torch.float32, device="cuda:0")
    c, s, _ = nv.quantize(to_dev(xh), offsets, global_scale=g)
    torch.cuda.synchronize()
    rc, rs, _ = orc.quantize(xh, *offsets, gscale=float(sg))
    gs, gc = to_host(s), to_host(c)
    assert np.array_equal(gs, rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc, rc), "codes: " + first_mismatch(gc, rc)


@pytest.mark.parametrize("offsets", [(-2, 6), (-8, 8)])
def test_mined_near_ties(gpu, orc, offsets):
    """The 1024 closest-call blocks out of 2^18 weight-style blocks."""
    xh = workloads.workload(4, (256, 16384))
    xf = workloads.bf16_bits_to_f32(xh).reshape(-1, 16)
    sg = np.float32(np.abs(xf).max() / np.float32(2688))
    gaps = _relative_gaps(xf, sg, *offsets)
    pick = np.argsort(gaps, kind="stable")[:1024]
    print(f"[near-ties] gaps of the picked blocks: min {gaps[pick].min():.2e} "
          f"max {gaps[pick].max():.2e}; exact ties {int((gaps[pick] == 0).sum())}")
    sel = xh.reshape(-1, 16)[pick].reshape(64, 256)
    check_given(gpu, orc, np.ascontiguousarray(sel), sg, offsets)


def test_perturbed_exact_ties(gpu, orc):
    """Grid-aligned blocks (several candidates reach SSE 0 or equal SSEs), each
    nudged by 0..3 bf16 ulps in one element."""
    rng = np.random.default_rng(11)
    n = 4096
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    vals = R.e4m3_values()
    p = rng.integers(24, 110, n)
    codes = rng.integers(0, 8, (n, 16))
    codes[:, 0] = 7  # amax on the grid maximum: the default pattern is p itself
    sign = rng.integers(0, 2, (n, 16)) * 2 - 1
    x = (sign * grid[codes] * vals[p][:, None]).astype(np.float32)
    xh = workloads.to_bf16_bits(x)
    bump = rng.integers(0, 4, n).astype(np.uint16)
    idx = rng.integers(1, 16, n)
    nz = (xh[np.arange(n), idx] & 0x7FFF) != 0
    xh[np.arange(n)[nz], idx[nz]] += bump[nz]
    for offsets in [(-2, 6), (-8, 8)]:
        check_given(gpu, orc, xh.reshape(-1, 256), np.float32(1.0), offsets)


@pytest.mark.parametrize("offsets", [(0, 0), (-1, 1), (-3, 2), (-8, 0), (0, 8), (-2, 6)])
def test_offset_subranges(gpu, orc, offsets):
    xh = workloads.workload(2, (96, 4096))
    xf = workloads.bf16_bits_to_f32(xh)
    sg = np.float32(np.abs(xf).max() / np.float32(2688))
    check_given(gpu, orc, xh, sg, offsets)


def test_magnitude_edges(gpu, orc):
    """Blocks just inside and outside [2^-40, 2^60], where the certificate stops applying."""
    base = workloads.bf16_bits_to_f32(workloads.workload(4, (8, 1024))) / np.float32(0.02)
    for e in (-45, -40, -39, 59, 60, 61):
        x = (base * np.float32(2.0 ** e)).astype(np.float32)
        xh = workloads.to_bf16_bits(x)
        xf = workloads.bf16_bits_to_f32(xh)
        sg = np.float32(np.abs(xf).max() / np.float32(2688))
        check_given(gpu, orc, xh, sg, (-2, 6))


# --- FP32 values: the certified search on three exact bf16 parts of each value ---

def test_mined_near_ties_f32(gpu, orc):
    """The 1024 closest-call blocks out of 2^17 FP32 Gaussian blocks (full 24-bit
    significands), offsets [-8, 8] and [-2, 6]."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((128, 16384)).astype(np.float32)
    xf = x.reshape(-1, 16)
    sg = np.float32(np.abs(xf).max() / np.float32(2688))
    for offsets in [(-2, 6), (-8, 8)]:
        gaps = _relative_gaps(xf, sg, *offsets)
        order = np.argsort(gaps, kind="stable")
        ties = order[gaps[order] == 0][:256]
        near = order[gaps[order] > 0][:1024 - ties.size]
        pick = np.concatenate([ties, near])
        print(f"[near-ties f32] {offsets}: {ties.size} exact ties, nonzero gaps "
              f"min {gaps[near].min():.2e} max {gaps[near].max():.2e}")
        sel = np.ascontiguousarray(xf[pick].reshape(64, 256))
        check_given(gpu, orc, sel, sg, offsets)


def test_twin_ties_f32(gpu, orc):
    """Blocks whose values sit inside the E2M1 cells {0, 1, 2, 3, 4, 6} of a pattern p
    (never the 0.5 or 1.5 cells) with the block maximum at 6..7 times its scale: the
    default pattern is p, p + 1 or p + 2, and the candidate at p and its twin at p + 8
    reconstruct every element alike (offset pairs (0, 8), (-1, 7), (-2, 6)); half of
    the blocks are then moved by 1..3 ulps in one element."""
    rng = np.random.default_rng(51)
    n = 8192
    vals = R.e4m3_values()
    p = rng.integers(40, 110, n)
    cells = np.array([[0.0, 0.24], [0.76, 1.24], [1.76, 2.49], [2.51, 3.49], [3.51, 4.99],
                      [5.01, 6.99]], np.float64)
    k = rng.integers(0, 6, (n, 16))
    v = rng.uniform(cells[k, 0], cells[k, 1])
    v[:, 0] = rng.uniform(6.0, 6.99, n)
    sign = rng.integers(0, 2, (n, 16)) * 2 - 1
    x = (sign * v * vals[p][:, None]).astype(np.float32)
    bits = x.view(np.uint32)
    idx = rng.integers(1, 16, n)
    bump = np.where(np.arange(n) % 2 == 0, 0, rng.integers(1, 4, n)).astype(np.uint32)
    nz = (bits[np.arange(n), idx] & 0x7FFFFFFF) != 0
    bits[np.arange(n)[nz], idx[nz]] += bump[nz]
    x = bits.view(np.float32)
    for offsets in [(-8, 8), (-2, 6)]:
        gaps = _relative_gaps(x, np.float32(1.0), *offsets)
        print(f"[twin ties] {offsets}: {int((gaps == 0).sum())} exact ties of {n}")
        assert (gaps == 0).sum() > (n // 8 if offsets == (-8, 8) else 40)
        check_given(gpu, orc, np.ascontiguousarray(x.reshape(-1, 256)), np.float32(1.0), offsets)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_identical_reconstructions(gpu, orc, dt):
    """Blocks whose values are V * s_p with V in {0, 1, 2, 3} and amax = 3 s_p: the
    default pattern is p - 8, and candidates p - 8 and p reconstruct every element
    alike (values doubled at half the scale), an exact tie the visiting order
    decides; half of the blocks nudged by a few ulps in one element."""
    rng = np.random.default_rng(31)
    n = 4096
    vals = R.e4m3_values()
    p = rng.integers(40, 110, n)
    V = np.array([0, 1, 2, 3], np.float32)[rng.integers(0, 4, (n, 16))]
    V[:, 0] = 3
    sign = rng.integers(0, 2, (n, 16)) * 2 - 1
    x = (sign * V * vals[p][:, None]).astype(np.float32)
    bits = x.view(np.uint32)
    idx = rng.integers(1, 16, n)
    bump = np.where(np.arange(n) % 2 == 0, 0, rng.integers(1, 4, n)).astype(np.uint32)
    nz = (bits[np.arange(n), idx] & 0x7FFFFFFF) != 0
    if dt == "bf16":
        xh = workloads.to_bf16_bits(x)
        xh[np.arange(n)[nz], idx[nz]] += bump[nz].astype(np.uint16)
        xin = xh.reshape(-1, 256)
    else:
        bits[np.arange(n)[nz], idx[nz]] += bump[nz]
        xin = bits.view(np.float32).reshape(-1, 256)
    for offsets in [(-8, 8), (0, 8), (-8, 0)]:
        check_given(gpu, orc, np.ascontiguousarray(xin), np.float32(1.0), offsets)


@pytest.mark.parametrize("offsets", [(0, 0), (-1, 1), (-3, 2), (-8, 0), (0, 8), (-8, 8)])
def test_offset_subranges_f32(gpu, orc, offsets):
    x = workloads.bf16_bits_to_f32(workloads.workload(2, (96, 4096)))
    x = (x * np.float32(1.0 + 2.0 ** -9)).astype(np.float32)  # full FP32 significands
    sg = np.float32(np.abs(x).max() / np.float32(2688))
    check_given(gpu, orc, x, sg, offsets)


def test_magnitude_edges_f32(gpu, orc):
    base = np.random.default_rng(41).standard_normal((8, 1024)).astype(np.float32)
    for e in (-45, -40, -39, 59, 60, 61):
        x = (base * np.float32(2.0 ** e)).astype(np.float32)
        sg = np.float32(np.abs(x).max() / np.float32(2688))
        check_given(gpu, orc, x, sg, (-2, 6))
        check_given(gpu, orc, x, sg, (-8, 8))


def test_default_pattern_near_e4m3_midpoints(gpu, orc):
    """The default pattern p0 = E4M3(fl(fl(amax / 6) / S_g)) where that quotient sits on or
    within a few ulps of an E4M3 rounding midpoint: block maxima on every bf16 significand
    over 18 binades, S_g = fl(2^j / 6) moved by -10..10 ulps, so the quotient is amax 2^-j
    up to a few ulps and every midpoint with five significant bits is met."""
    rng = np.random.default_rng(31)
    sig = np.arange(128, 256, dtype=np.float32) / np.float32(128)
    am = np.concatenate([sig * np.float32(2.0 ** e) for e in range(-8, 10)]).astype(np.float32)
    rest = (rng.uniform(-1, 1, (am.size, 15)) * am[:, None]).astype(np.float32)
    xh = workloads.to_bf16_bits(np.concatenate([am[:, None], rest], 1)).reshape(-1, 1024)
    amax = np.abs(workloads.bf16_bits_to_f32(xh)).reshape(-1, 16).max(1)
    near = ties = 0
    for j in (0, 3):
        base = int(np.array([2.0 ** j / 6], np.float32).view(np.uint32)[0])
        for k in range(-10, 11):
            sg = np.array([base + k], np.uint32).view(np.float32)[0]
            t = ((amax / np.float32(6)).astype(np.float32) / sg).astype(np.float32)
            tb = t.view(np.uint32).astype(np.int64)
            normal = (t >= 2.0 ** -6) & (t < 448)
            near += int(np.sum(normal & (((tb - 0x80000 + 8) & 0xFFFFF) <= 16)))
            ties += int(np.sum(normal & ((tb & 0xFFFFF) == 0x80000)))
            for offsets in [(0, 0), (-2, 6)]:
                check_given(gpu, orc, xh, sg, offsets)
    print(f"[p0] blocks within 8 ulps of an E4M3 midpoint: {near}, exactly on one: {ties}")
    assert near > 1000 and ties > 100


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_saturating_given_scale(gpu, orc, dt):
    """A caller-given tensor scale 2^1 .. 2^7 below amax / 2688 (rows of widely
    different magnitudes): the default patterns of the larger blocks saturate at
    448, where the certificate's bounds do not hold, so those blocks take the
    exact search."""
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((64, 1024)) * np.exp(rng.normal(0.0, 1.5, (64, 1)))).astype(np.float32)
    xin = workloads.to_bf16_bits(x) if dt == "bf16" else x
    xf = workloads.bf16_bits_to_f32(xin) if dt == "bf16" else x
    amax = np.abs(xf).reshape(-1, 16).max(1)
    A = float(np.abs(xf).max())
    for k in (1, 3, 7):
        sg = np.float32(A / 2688.0 / 2.0 ** k)
        t = ((amax / np.float32(6)).astype(np.float32) / sg).astype(np.float32)
        print(f"[saturating] {dt} S_g = A / 2688 / 2^{k}: {int((t > 448).sum())} of {amax.size} "
              "blocks saturated")
        assert (t > 448).sum() > 0 and (t <= 447).sum() > 0
        for offsets in [(-2, 6), (-8, 8)]:
            check_given(gpu, orc, np.ascontiguousarray(xin), sg, offsets)
