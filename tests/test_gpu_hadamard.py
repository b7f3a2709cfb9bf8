"""GPU checks of the 128-point Hadamard pre-transform on MFMA (ScaleSearch summary
page, ScaleSearchAttention, 非干渉処理（IP）と絶対値低減).

The MFMA accumulates in FP32, so the transform may differ from the oracle's
exactly rounded one by a few FP32 ulps. Bars:
  - before coding: per vector max |y - y_ref| <= 1e-5 * max |y_ref|, and the
    normalized absolute error mean|y - y_ref| / mean|y_ref| <= 1e-5;
  - split parity: the oracle's quantizer fed the GPU's own FP32 transform gives
    the GPU's codes, scales and tensor scale bit for bit;
  - end to end: blocks whose codes or scale differ from the oracle's are at
    most 1e-4 of all blocks.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def check_transform(y, ref):
    y = y.reshape(-1, 128).astype(np.float64)
    ref = ref.reshape(-1, 128).astype(np.float64)
    vmax = np.abs(ref).max(axis=1)
    dev = np.abs(y - ref).max(axis=1)
    assert np.all(dev <= 1e-5 * vmax + 1e-30), f"worst {np.max(dev / np.maximum(vmax, 1e-30))}"
    nae = np.abs(y - ref).mean() / max(np.abs(ref).mean(), 1e-30)
    assert nae <= 1e-5, nae
    return float(np.mean(y == ref)), nae


def test_closed_forms(gpu):
    x = np.zeros((64, 128), np.float32)
    x[0, :] = 1.0
    x[1, 5] = 1.0
    x[2, 0] = -2.0
    for r in range(3, 64):
        x[r, r] = float(r)
    xb = workloads.to_bf16_bits(x)
    y = to_host(gpu.hadamard128(to_dev(xb)))
    assert y[0, 0] == np.float32(np.sqrt(128.0)) and np.all(y[0, 1:] == 0)
    c32 = np.float32(np.sqrt(1.0 / 128.0))  # binary32 nearest 2^-3.5, the kernel's scale
    assert np.all(np.abs(y[1]) == c32)
    # a single nonzero input: every output is +-x times that scale, one binary32 rounding
    for r in range(3, 64):
        assert np.all(np.abs(y[r]) == np.float32(np.float32(r) * c32))


@pytest.mark.parametrize("shape", [(1, 2, 333, 128), (5, 256), (1, 1, 31, 128), (3, 1024)])
def test_transform_within_tolerance(gpu, orc, shape):
    x = workloads.workload(5, shape)
    y = to_host(gpu.hadamard128(to_dev(x)))
    exact, nae = check_transform(y, orc.hadamard128(x))
    print(f"[hadamard] {shape}: {exact:.4f} of outputs bit-exact, NAE {nae:.2e}")


def _split_and_end_to_end(nv, orc, x, offsets=(-8, 8)):
    xd = to_dev(x)
    c, s, g = nv.quantize(xd, offsets, hadamard=True)
    y = nv.hadamard128(xd)
    torch.cuda.synchronize()
    gc, gs, gg = to_host(c), to_host(s), np.float32(to_host(g)[0])
    yh = to_host(y).reshape(-1, x.shape[-1])
    # split parity: oracle quantizer on the GPU's own transform
    rc, rs, rg = orc.quantize(yh, *offsets)
    assert gg == rg
    assert np.array_equal(gs.reshape(rs.shape), rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc.reshape(rc.shape), rc), "codes: " + first_mismatch(gc, rc)
    # end to end against the oracle's exactly rounded transform
    ec, es, eg = orc.quantize(x.reshape(-1, x.shape[-1]), *offsets, hadamard=True)
    assert abs(float(gg) - float(eg)) <= 1e-5 * float(eg)
    bad = (es != gs.reshape(es.shape)) | np.any(
        ec.reshape(-1, 8) != gc.reshape(-1, 8), axis=1).reshape(es.shape)
    frac = bad.mean()
    print(f"[hadamard] {x.shape}: {bad.sum()} of {bad.size} blocks differ end to end ({frac:.2e})")
    assert frac <= 1e-4
    return c, s, g


@pytest.mark.parametrize("shape", [(1, 4, 2048, 128), (7, 384), (1, 1, 33, 128)])
def test_quantize_hadamard_shrunk(gpu, orc, shape):
    _split_and_end_to_end(gpu, orc, workloads.workload(5, shape))


def test_quantize_hadamard_full(gpu, orc):
    """Workload 5 at full size: bf16 Q [1, 32, 32768, 128], offsets [-8, 8]; the
    transform itself against the oracle's over the whole tensor, in chunks of four
    heads."""
    x = workloads.workload(5)
    _split_and_end_to_end(gpu, orc, x)
    xd = to_dev(x)
    worst_exact = 1.0
    for h0 in range(0, 32, 4):
        y = to_host(gpu.hadamard128(xd[:, h0:h0 + 4].contiguous()))
        exact, _ = check_transform(y, orc.hadamard128(np.ascontiguousarray(x[:, h0:h0 + 4])))
        worst_exact = min(worst_exact, exact)
    print(f"[hadamard] full tensor within 1e-5; lowest bit-exact share of a chunk {worst_exact:.4f}")


def test_hadamard_global_scale_entry_point(gpu, orc):
    x = workloads.workload(5, (1, 2, 500, 128))
    xd = to_dev(x)
    g = gpu.global_scale(xd, hadamard=True)
    y = gpu.hadamard128(xd)
    torch.cuda.synchronize()
    _, _, rg = orc.quantize(to_host(y).reshape(-1, 128), 0, 0)
    assert np.float32(g.item()) == rg


def test_hadamard_sink_mode(gpu, orc):
    kv = workloads.workload(3, (1, 3, 700, 128))
    kvd = to_dev(kv)
    c, s, g, sink = gpu.quantize_kv_sink(kvd, 128, 128, (-8, 8), hadamard=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(sink)[:, :, :128], kv[:, :, :128])
    # split parity on the middle tokens
    mid = kvd[:, :, 128:700 - 128].contiguous()
    y = to_host(gpu.hadamard128(mid)).reshape(-1, 128)
    rc, rs, rg = orc.quantize(y, -8, 8)
    assert np.float32(to_host(g)[0]) == rg
    assert np.array_equal(to_host(s).reshape(rs.shape), rs)
    assert np.array_equal(to_host(c).reshape(rc.shape), rc)


def test_hadamard_non_finite(gpu, orc):
    x = workloads.workload(5, (2, 256))
    x[1, 7] = 0x7F80  # +Inf in bf16
    c, s, g = gpu.quantize(to_dev(x), (-8, 8), hadamard=True)
    torch.cuda.synchronize()
    assert np.isnan(g.item())
    assert np.all(to_host(s) == 0x7F) and np.all(to_host(c) == 0)


def test_hadamard_saturating_given_scale(gpu, orc):
    """The Hadamard path with a caller-given tensor scale 2^4 below the transform's
    amax / 2688: the blocks whose default pattern saturates take the exact search.
    Split parity: the oracle quantizes the GPU's own transform under the same S_g."""
    x = workloads.workload(5, (1, 2, 300, 128))
    xd = to_dev(x)
    y = to_host(gpu.hadamard128(xd)).reshape(-1, 128)
    sg = np.float32(np.abs(y).max() / 2688.0 / 16.0)
    g = torch.tensor([sg], dtype=torch.float32, device="cuda:0")
    for offsets in [(-8, 8), (-2, 6)]:
        c, s, _ = gpu.quantize(xd, offsets, hadamard=True, global_scale=g)
        torch.cuda.synchronize()
        rc, rs, _ = orc.quantize(y, *offsets, gscale=float(sg))
        assert np.array_equal(to_host(s).reshape(rs.shape), rs)
        assert np.array_equal(to_host(c).reshape(rc.shape), rc)
