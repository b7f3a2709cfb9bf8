"""GPU parity of the attention-sink KV mode (ScaleSearch summary page,
ScaleSearchAttention, アテンション・シンク対応混合精度キャッシング): first and last
tokens of every (batch, head) kept verbatim, the middle quantized with a tensor
scale from the middle tokens only. Compared bit for bit with the oracle."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same_floats, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def check_sink(nv, orc, kv_np, nf, nl, offsets=(-2, 6)):
    print(f"[case] kv={kv_np.shape} {kv_np.dtype} sink={nf}+{nl} offsets={offsets}", flush=True)
    kv = to_dev(kv_np)
    c, s, g, sink = nv.quantize_kv_sink(kv, nf, nl, offsets)
    torch.cuda.synchronize()
    rc, rs, rg, rsink = orc.quantize_kv_sink(kv_np, nf, nl, *offsets)
    assert np.float32(to_host(g)[0]) == rg
    gs, gc = to_host(s), to_host(c)
    assert np.array_equal(gs, rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc, rc), "codes: " + first_mismatch(gc, rc)
    assert np.array_equal(to_host(sink), rsink)
    T = kv_np.shape[2]
    for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        y = to_host(nv.dequantize_kv_sink(c, s, g, sink, T, nf, nl, tdt))
        ref = orc.dequantize_kv_sink(rc, rs, rg, rsink, T, nf, nl, out)
        assert_same_floats(y, ref)


@pytest.mark.parametrize("shape,nf,nl", [
    ((1, 8, 2048, 128), 128, 128),
    ((2, 3, 300, 128), 20, 17),
    ((1, 2, 256, 128), 128, 128),   # nothing in the middle
    ((1, 2, 300, 64), 0, 0),        # nothing kept aside
    ((1, 1, 5, 16), 1, 3),
    ((3, 1, 200, 32), 0, 50),
])
def test_sink_parity_shrunk(gpu, orc, shape, nf, nl):
    check_sink(gpu, orc, workloads.workload(3, shape), nf, nl)


def test_sink_fp32(gpu, orc):
    kv = workloads.bf16_bits_to_f32(workloads.workload(3, (1, 4, 400, 128)))
    check_sink(gpu, orc, kv, 128, 128)


def test_sink_parity_full(gpu, orc):
    check_sink(gpu, orc, workloads.workload(3), 128, 128)


def test_sink_middle_equals_plain_quantize(gpu):
    kvn = workloads.workload(3, (1, 4, 1024, 128))
    kv = to_dev(kvn)
    c, s, g, sink = gpu.quantize_kv_sink(kv, 128, 128)
    mid = kv[:, :, 128:1024 - 128].contiguous()
    c2, s2, g2 = gpu.quantize(mid)
    torch.cuda.synchronize()
    assert torch.equal(g, g2) and torch.equal(c, c2) and torch.equal(s, s2)
