"""GPU parity of the MXFP4 contrast format (32-element blocks, E8M0 scales; read as
the OCP Microscaling format, set against NVFP4 on "NVIDIAのFP4推論が50倍の効率を実現",
超低精度推論を支えるアーキテクチャ), with and without the exponent search carried over
from the ScaleSearch summary page. Bit for bit against the oracle: codes, scale
bytes and dequantized values."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same_floats, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def check(gpu, orc, x, offsets=(0, 0), deq=True):
    print(f"[case] mxfp4 shape={x.shape} dtype={x.dtype} offsets={offsets}", flush=True)
    c, s = gpu.mxfp4_quantize(to_dev(x), offsets)
    torch.cuda.synchronize()
    gc, gs = to_host(c), to_host(s)
    rc, rs = orc.quantize_mxfp4(x, *offsets)
    assert np.array_equal(gs, rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc, rc), "codes: " + first_mismatch(gc, rc)
    if deq:
        for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            y = to_host(gpu.mxfp4_dequantize(c, s, tdt))
            assert_same_floats(y, orc.dequantize_mxfp4(rc, rs, out))
    return gc, gs


@pytest.mark.parametrize("idx,shape", [(1, (333, 1024)), (2, (517, 4096)), (3, (1, 3, 701, 128)),
                                       (4, (129, 28672)), (5, (1, 2, 999, 128))])
@pytest.mark.parametrize("offsets", [(0, 0), (-1, 1), (-3, 3)])
def test_workloads_shrunk(gpu, orc, idx, shape, offsets):
    check(gpu, orc, workloads.workload(idx, shape), offsets)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_special_values(gpu, orc, dt):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, 5] = np.inf
    x[3, 40] = np.nan
    x[4, :32] = 1e-44                       # subnormal block
    x[5, :32] = np.float32(3.0e38)          # near the top of the range
    x[6, 64:96] = np.linspace(-7.9, 7.9, 32)  # amax in (6, 8): clipping at X = 0
    x[7, :32] = np.float32(2.0 ** -126) * np.arange(32)
    x[8, :] = np.float32(2.0 ** 127)
    if dt == "bf16":
        x = workloads.to_bf16_bits(x)
    for offsets in [(0, 0), (-1, 1), (-8, 8)]:
        check(gpu, orc, x, offsets)


def test_dequantize_every_byte(gpu, orc):
    """Every scale byte (255 = NaN) and every code nibble."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, (256, 64), dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1).repeat(4, axis=1)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        y = to_host(gpu.mxfp4_dequantize(cd, sd, tdt))
        assert_same_floats(y, orc.dequantize_mxfp4(codes, scales, out))


def test_empty_and_full(gpu, orc):
    c, s = gpu.mxfp4_quantize(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda:0"))
    assert c.shape == (0, 32) and s.shape == (0, 2)
    x = workloads.workload(4)
    for offsets in [(0, 0), (-1, 1)]:
        check(gpu, orc, x, offsets, deq=False)
