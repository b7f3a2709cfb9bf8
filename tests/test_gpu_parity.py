"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for bit.

Codes, scales, the tensor scale and dequantized values must be identical to
the oracle's on the same seeded inputs (workload recipes of the workloads
module), at sizes spanning many workgroups with ragged tails and at the full
workload sizes the benchmark times.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same_floats, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_gpu(nv, x_np, offsets, gscale=None):
    x = to_dev(x_np)
    g_in = None if gscale is None else torch.tensor([gscale], dtype=torch.float32, device=x.device)
    c, s, g = nv.quantize(x, offsets, global_scale=g_in)
    torch.cuda.synchronize()
    return to_host(c), to_host(s), np.float32(to_host(g)[0]), (c, s, g)


def check_quantize(nv, orc, x_np, offsets=(-2, 6), gscale=None, deq=True):
    print(f"[case] shape={x_np.shape} dtype={x_np.dtype} offsets={offsets} gscale={gscale}",
          flush=True)
    gc, gs, gg, dev = run_gpu(nv, x_np, offsets, gscale)
    rc, rs, rg = orc.quantize(x_np, *offsets, gscale=gscale)
    assert f"{gg!r}" == f"{rg!r}" or (np.isnan(gg) and np.isnan(rg)), (gg, rg)
    assert np.array_equal(gs, rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc, rc), "codes: " + first_mismatch(gc, rc)
    if deq:
        c, s, g = dev
        for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            y = to_host(nv.dequantize(c, s, g, tdt))
            assert_same_floats(y, orc.dequantize(rc, rs, rg, out))
    return gc, gs, gg


# --- the hardware E2M1 convert, exercised through the quantizer --------------

def _window(v, n):
    u = np.array([v], np.float32).view(np.uint32)[0].astype(np.int64)
    return np.arange(max(u - n, 0), u + n + 1, dtype=np.int64).astype(np.uint32).view(np.float32)


def test_e2m1_convert_through_quantizer(gpu, orc):
    """Blocks [6, v1..v15] under S_g = 1 get scale 1.0 (pattern 0x38), so with offsets
    [0, 0] every code is the E2M1 rounding of v itself: midpoints, ulp windows around
    them, both signs, signed zeros and subnormals."""
    vals = [_window(m, 2048) for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0)]
    vals.append(np.array([0.0, 1e-45, 1e-40, 1.1754942e-38, 1e-30, 0.2, 5.999, 6.0], np.float32))
    v = np.concatenate(vals)
    v = np.concatenate([v, -v])
    v = v[np.abs(v) <= 6.0]
    n = -(-v.size // 15) * 15
    v = np.concatenate([v, np.zeros(n - v.size, np.float32)]).reshape(-1, 15)
    x = np.concatenate([np.full((v.shape[0], 1), 6.0, np.float32), v], axis=1)
    x = np.ascontiguousarray(x.reshape(-1, 64) if x.size % 64 == 0 else
                             np.concatenate([x.reshape(-1), np.zeros((-x.size) % 64, np.float32)])
                             .reshape(-1, 64))
    for offs in [(0, 0), (-2, 6)]:
        gc, gs, gg = check_quantize(gpu, orc, x, offs, gscale=1.0)
    assert gg == 1.0


def test_saturation_and_tiny_scales(gpu, orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    # given tensor scales far from the data: saturating and underflowing candidates
    for g in (1e-30, 1e-6, 3.0, 1e10, 1e30):
        check_quantize(gpu, orc, x, (-8, 8), gscale=g)


# --- workloads ------------------------------------------------------------------

SHRUNK = [
    (1, (1024, 1024), (-2, 6)),
    (1, (77, 1024), (-2, 6)),
    (1, (3, 48), (-2, 6)),
    (2, (333, 4096), (-2, 6)),
    (4, (97, 28672), (-2, 6)),
    (4, (256, 28672 // 7 // 16 * 16), (0, 0)),
    (2, (64, 4096), (-8, 8)),
    (1, (65, 1024), (-126, 126)),
    (2, (31, 4096), (-1, 3)),
]


@pytest.mark.parametrize("idx,shape,offs", SHRUNK)
def test_workload_parity_shrunk(gpu, orc, idx, shape, offs):
    check_quantize(gpu, orc, workloads.workload(idx, shape), offs)


@pytest.mark.parametrize("idx", [1, 2])
def test_workload_parity_full(gpu, orc, idx):
    w = workloads.WORKLOADS[idx]
    check_quantize(gpu, orc, workloads.workload(idx), w["offsets"])


def test_workload4_full_size(gpu, orc):
    """The benchmark's workload: bf16 8192 x 28672, offsets [-2, 6], full compare."""
    x = workloads.workload(4)
    check_quantize(gpu, orc, x, (-2, 6), deq=False)
    # dequantize (bf16 out, the benchmark's) compared on every row, 1024 rows at a time
    xd = to_dev(x)
    c, s, g = gpu.quantize(xd, (-2, 6))
    y = gpu.dequantize(c, s, g, torch.bfloat16)
    torch.cuda.synchronize()
    hc, hs, sg = to_host(c), to_host(s), np.float32(to_host(g)[0])
    for r0 in range(0, 8192, 1024):
        ref = orc.dequantize(hc[r0:r0 + 1024], hs[r0:r0 + 1024], sg, "bf16")
        assert_same_floats(to_host(y[r0:r0 + 1024]), ref)


# --- edge cases ---------------------------------------------------------------------

def test_empty_tensor(gpu):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda:0")
    c, s, g = gpu.quantize(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 32) and s.shape == (0, 4)
    assert g.item() == 1.0


def test_all_zero_and_negative_zero(gpu, orc):
    x = np.zeros((5, 64), np.float32)
    x[2] = -0.0
    check_quantize(gpu, orc, x)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_contract(gpu, orc, bad):
    x = workloads.workload(1, (40, 1024))
    x[17, 333] = bad
    check_quantize(gpu, orc, x)
    check_quantize(gpu, orc, x, gscale=0.001)  # given scale: only that block


def test_given_scale_equals_computed(gpu, orc):
    x = workloads.workload(2, (128, 4096))
    _, _, g = check_quantize(gpu, orc, x)
    check_quantize(gpu, orc, x, gscale=float(g))


def test_tiny_huge_and_subnormal_tensors(gpu, orc):
    base = workloads.workload(1, (32, 256)).astype(np.float64)
    for sc in (1e-38, 1e-42, 1e-20, 1e25, 1e37):
        check_quantize(gpu, orc, (base * sc).astype(np.float32))


def test_grid_aligned_round_trip(gpu, orc):
    rng = np.random.default_rng(7)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    p = rng.integers(16, 120, 4096)
    sv = np.array([orc.e4m3_value(int(q)) for q in p], np.float32)
    x = (grid[rng.integers(0, 8, (4096, 16))] * sv[:, None] *
         (rng.integers(0, 2, (4096, 16)) * 2 - 1)).astype(np.float32)
    x[0] = 0
    x[0, 0] = 2688.0
    check_quantize(gpu, orc, x.reshape(-1, 256))


def test_determinism_and_streams(gpu):
    x = to_dev(workloads.workload(2, (512, 4096)))
    c1, s1, g1 = gpu.quantize(x)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c2, s2, g2 = gpu.quantize(x)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(g1, g2)


def test_global_scale_entry_point(gpu, orc):
    x = workloads.workload(2, (256, 4096))
    g = gpu.global_scale(to_dev(x))
    torch.cuda.synchronize()
    _, _, rg = orc.quantize(x, 0, 0)
    assert np.float32(g.item()) == rg


def test_dequantize_every_code_and_scale(gpu, orc):
    codes = np.tile(np.arange(256, dtype=np.uint8), 64).reshape(128, 128)
    scales = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(128, 16)
    for g in (1.0, 0.00123, 3.5e-39, 1e30, float("nan")):
        gd = torch.tensor([g], dtype=torch.float32, device="cuda:0")
        for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            y = to_host(gpu.dequantize(to_dev_u8(codes), to_dev_u8(scales), gd, tdt))
            assert_same_floats(y, orc.dequantize(codes, scales, np.float32(g), out))


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def test_e2m1_convert_strided_sweep(gpu, orc):
    """Every 97th binary32 bit pattern in [0, 6] (about 11 million values: every exponent,
    mantissa patterns in steps of 97 ulps), both signs, through the quantizer as above."""
    top = int(np.array([6.0], np.float32).view(np.uint32)[0])
    v = np.arange(0, top + 1, 97, dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, -v])
    n = -(-v.size // 15) * 15
    v = np.concatenate([v, np.zeros(n - v.size, np.float32)]).reshape(-1, 15)
    blocks = np.concatenate([np.full((v.shape[0], 1), 6.0, np.float32), v], axis=1)
    pad = (-blocks.shape[0]) % 64
    blocks = np.concatenate([blocks, np.zeros((pad, 16), np.float32)])
    x = np.ascontiguousarray(blocks.reshape(-1, 1024))
    check_quantize(gpu, orc, x, (0, 0), gscale=1.0, deq=False)


def test_random_shapes_and_values(gpu, orc):
    """Seeded random shapes (rows 1..257, cols 16..4096), dtypes, magnitudes, offset ranges
    (the certified ranges and, every sixth case, one beyond +-8 for the exact search) and
    special values: zero blocks, signed zeros, an outlier, a subnormal block."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        rows, cols = int(rng.integers(1, 258)), 16 * int(rng.integers(1, 257))
        x = (rng.standard_normal((rows, cols)) * np.float32(np.exp(rng.uniform(-20, 20))))
        x = x.astype(np.float32)
        r, c = int(rng.integers(0, rows)), 16 * int(rng.integers(0, cols // 16))
        kind = case % 5
        if kind == 0:
            x[r, c:c + 16] = 0.0
        elif kind == 1:
            x[r, c:c + 16] = -0.0
        elif kind == 2:
            x[r, c] *= np.float32(1e6)
        elif kind == 3:
            x[r, c:c + 16] = np.float32(1e-40) * np.arange(16, dtype=np.float32)
        lo, hi = -int(rng.integers(0, 9)), int(rng.integers(0, 9))
        if case % 6 == 5:
            lo, hi = -12, 10
        xin = workloads.to_bf16_bits(x) if case % 2 == 0 else x
        check_quantize(gpu, orc, xin, (lo, hi))
