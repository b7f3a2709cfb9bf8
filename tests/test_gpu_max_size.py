"""GPU parity at the largest tensor the C ABI accepts: 2^29 blocks of 16.

bf16 [524288, 16384] (17.2 GB) and FP32 of the same shape (34.4 GB), so that the
kernels' 32-bit block and 16-byte-chunk indices reach the top of their range
(2^29 blocks; 2^31 chunks for the FP32 input and output). The input is drawn on
the device (8.6 G values are too many to draw on the host in a test) by the
seeded generator of the workloads module, with its largest magnitude planted in
the last row, so the oracle, given sampled rows that include that row, derives
the same tensor scale from them alone. The sampled rows (the first four, the last
four and 24 seeded ones between) are compared bit for bit: codes, scales, tensor
scale and dequantized values.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same_floats, first_mismatch, to_host

pytestmark = pytest.mark.gpu

ROWS, COLS = 524288, 16384  # 2^29 blocks of 16: the ABI's limit


def _sample_rows(seed: int) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(4, ROWS - 4), size=24, replace=False)
    idx = np.unique(np.concatenate([np.arange(4), np.arange(ROWS - 4, ROWS), mid]))
    return torch.from_numpy(idx.astype(np.int64))


def _max_tensor(dtype, seed: int) -> torch.Tensor:
    print(f"[case] max size {ROWS}x{COLS} {dtype} seed {seed}", flush=True)
    return workloads.device_gaussian_planted(ROWS, COLS, seed, dtype, "cuda:0")


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,deq", [(torch.bfloat16, torch.bfloat16),
                                       (torch.float32, torch.float32)], ids=["bf16", "fp32"])
def test_quantize_and_dequantize_at_the_limit(gpu, orc, dtype, deq):
    x = _max_tensor(dtype, 11 if dtype == torch.bfloat16 else 12)
    try:
        c, s, g = gpu.quantize(x, (-2, 6))
        y = gpu.dequantize(c, s, g, deq)
        idx = _sample_rows(13).to(x.device)
        xs = to_host(x.index_select(0, idx))
        cs, ss = to_host(c.index_select(0, idx)), to_host(s.index_select(0, idx))
        ys = to_host(y.index_select(0, idx))
        gg = np.float32(to_host(g)[0])
        del c, s, y
    finally:
        del x
        _free()
    rc, rs, rg = orc.quantize(xs, -2, 6)
    assert rg == np.float32(np.float32(8.0) / np.float32(2688.0))
    assert f"{gg!r}" == f"{rg!r}", (gg, rg)
    assert np.array_equal(ss, rs), "scales: " + first_mismatch(ss, rs)
    assert np.array_equal(cs, rc), "codes: " + first_mismatch(cs, rc)
    assert_same_floats(ys, orc.dequantize(rc, rs, rg, "bf16" if deq == torch.bfloat16 else "f32"))


def test_hadamard_quantize_at_the_limit(gpu, orc):
    """The fused Hadamard quantize (offsets [-8, 8], a given tensor scale) at 2^29
    blocks; the sampled rows against the oracle quantizer on the GPU's own FP32
    transform of those rows (the transform is per 128-vector, so those rows alone
    give the values the fused kernel codes)."""
    x = _max_tensor(torch.bfloat16, 14)
    gs = torch.tensor([0.004], dtype=torch.float32, device=x.device)
    try:
        c, s, _ = gpu.quantize(x, (-8, 8), hadamard=True, global_scale=gs)
        idx = _sample_rows(15).to(x.device)
        t = to_host(gpu.hadamard128(x.index_select(0, idx)))
        cs, ss = to_host(c.index_select(0, idx)), to_host(s.index_select(0, idx))
        del c, s
    finally:
        del x
        _free()
    rc, rs, _ = orc.quantize(t, -8, 8, gscale=np.float32(0.004))
    assert np.array_equal(ss, rs), "scales: " + first_mismatch(ss, rs)
    assert np.array_equal(cs, rc), "codes: " + first_mismatch(cs, rc)
