"""The Python binding refuses caller tensors the kernels could read or write out of
bounds (wrong shape, dtype, device or layout) before anything is launched, and
accepts the right ones."""
import numpy as np
import pytest
import torch

import microscaling_fp4_block_amd as nv
import workloads
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def test_dequantize_out_and_scale_checks(gpu):
    x = to_dev(workloads.workload(4, (8, 256)))
    c, s, g = nv.quantize(x)
    y = nv.dequantize(c, s, g, torch.bfloat16)
    out = torch.empty_like(y)
    assert torch.equal(nv.dequantize(c, s, g, out=out), y)  # right out: same result
    with pytest.raises(ValueError):
        nv.dequantize(c, s, g, out=torch.empty(8, 128, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        nv.dequantize(c, s, g, out=torch.empty(8, 512, dtype=torch.bfloat16, device="cuda")[:, ::2])
    with pytest.raises(ValueError):
        nv.dequantize(c, s[:, :-1].contiguous(), g)
    with pytest.raises(ValueError):
        nv.dequantize(c, s, g.cpu())
    with pytest.raises(ValueError):
        nv.dequantize(c, s, torch.ones(2, device="cuda"))


def test_workspace_and_given_scale_checks(gpu):
    x = to_dev(workloads.workload(4, (8, 256)))
    with pytest.raises(ValueError):
        nv.quantize(x, workspace=torch.empty(4096, dtype=torch.uint8))  # host memory
    with pytest.raises(ValueError):
        nv.quantize(x, global_scale=torch.ones(1))
    ws = torch.empty(1024, dtype=torch.int32, device="cuda")  # 4096 bytes of any dtype
    c0, s0, g0 = nv.quantize(x)
    c1, s1, g1 = nv.quantize(x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(g0, g1)
    kv = to_dev(workloads.workload(3, (1, 2, 300, 128)))
    with pytest.raises(ValueError):
        nv.quantize_kv_sink(kv, 16, 16, global_scale=torch.ones(1))
    with pytest.raises(ValueError):
        nv.quantize_kv_sink(kv, 16, 16, workspace=torch.empty(4096, dtype=torch.uint8))


def test_kv_sink_and_cache_shape_checks(gpu):
    kv = to_dev(workloads.workload(3, (1, 2, 300, 128)))
    c, s, g, sink = nv.quantize_kv_sink(kv, 16, 16)
    with pytest.raises(ValueError):
        nv.dequantize_kv_sink(c[:, :, :-1].contiguous(), s, g, sink, 300, 16, 16)
    with pytest.raises(ValueError):
        nv.dequantize_kv_sink(c, s, g, sink, 20, 16, 16)  # T below the sink size
    cache = nv.kv_cache_alloc(1, 2, 128, 400, 16, 16)
    bad = dict(cache, head=torch.empty(1, 2, 8, 128, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        nv.kv_append(bad, kv, g)
    with pytest.raises(ValueError):
        nv.kv_append(cache, kv.float(), g)  # dtype differs from the cache


def test_attention_operand_checks(gpu, orc):
    x = to_dev(workloads.workload(3, (1, 2, 64, 128)))
    q = nv.quantize(x)
    k = nv.quantize(x[:, :1].contiguous())
    with pytest.raises(ValueError):
        nv.attention((q[0], q[1][..., :4].contiguous(), q[2]), k, k)
    with pytest.raises(ValueError):
        nv.attention(q, k, (k[0], k[1], k[2].cpu()))
    cache = nv.kv_cache_alloc(1, 1, 128, 128, 16, 16)
    g = nv.global_scale(x)
    nv.kv_append(cache, x[:, :1].contiguous(), g)
    bad = dict(cache, tail=torch.empty(1, 1, 8, 128, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        nv.attention_kv_cache(q, cache, g, bad, g)
    o = nv.attention_kv_cache(q, cache, g, cache, g)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 64, 128) and torch.isfinite(o).all()
    # split keys: a piece size that is not a whole number of 32-key tiles, and a
    # workspace one byte short, are refused before any launch
    with pytest.raises(ValueError):
        nv.attention_kv_cache(q, cache, g, cache, g, split=48)
    need = nv.attention_split_workspace_bytes(1, 2, 64, cache["codes"].shape[2], 32)
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        nv.attention_kv_cache(q, cache, g, cache, g, split=32, workspace=short)
    o2 = nv.attention_kv_cache(q, cache, g, cache, g, split=32,
                               workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert o2.shape == (1, 2, 64, 128) and torch.isfinite(o2).all()


def test_mxfp4_out_checks(gpu):
    x = to_dev(workloads.workload(4, (8, 256)))
    c, s = nv.mxfp4_quantize(x)
    with pytest.raises(ValueError):
        nv.mxfp4_dequantize(c, s, out=torch.empty(8, 128, device="cuda"))
    with pytest.raises(ValueError):
        nv.mxfp4_dequantize(c, s[:, :-1].contiguous())
