"""GPU parity at the largest tensor the C ABI accepts: 2^29 blocks of 16.

bf16 [524288, 16384] (17.2 GB) and FP32 of the same shape (34.4 GB), so that the
kernels' 32-bit block and 16-byte-chunk indices reach the top of their range
(2^29 blocks; 2^31 chunks for the FP32 input and output), and the attention-sink
mode on a bf16 KV tensor [1, 8, 2^23, 128] of the same size, whose row map divides
block indices by the blocks per row and the middle tokens per head; MXFP4 (2^28
blocks of 32) on the bf16 tensor; and a decode append into the last row of a KV
cache of 2^23 tokens per head (8 heads), the most the ABI accepts. The input is drawn on
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
from gpu_util import assert_same_floats, first_mismatch, to_dev, to_host

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


def test_sink_mode_at_the_limit(gpu, orc):
    """Sink mode (128 + 128 tokens kept) on bf16 [1, 8, 8388608, 128], 2^29 blocks, the
    largest magnitude planted in the last middle token of the last head (the amax is
    taken over the middle tokens only). Sampled middle tokens of three heads against
    the oracle quantizer on those tokens; the kept tokens against the input; the
    reassembled dequantize (bf16) on the same tokens."""
    H, T, D, nf, nl = 8, 1 << 23, 128, 128, 128
    print(f"[case] sink mode at the limit [1, {H}, {T}, {D}]", flush=True)
    planted = (H - 1) * T + (T - nl - 1)
    kv = workloads.device_gaussian_planted(H * T, D, 16, torch.bfloat16, "cuda:0",
                                           row=planted).view(1, H, T, D)
    rng = np.random.default_rng(17)
    toks = np.unique(np.concatenate([[nf, nf + 1, T // 2, T - nl - 2, T - nl - 1],
                                     rng.integers(nf, T - nl, size=11)]))
    heads = [0, 3, H - 1]
    try:
        c, s, g, sink = gpu.quantize_kv_sink(kv, nf, nl, (-2, 6))
        y = gpu.dequantize_kv_sink(c, s, g, sink, T, nf, nl, torch.bfloat16)
        ti = torch.from_numpy(toks.astype(np.int64)).to(kv.device)
        ki = torch.from_numpy(np.concatenate([np.arange(nf), np.arange(T - nl, T)])).to(kv.device)
        xs = np.stack([to_host(kv[0, h].index_select(0, ti)) for h in heads])
        cs = np.stack([to_host(c[0, h].index_select(0, ti - nf)) for h in heads])
        ss = np.stack([to_host(s[0, h].index_select(0, ti - nf)) for h in heads])
        ys = np.stack([to_host(y[0, h].index_select(0, ti)) for h in heads])
        kept_in = np.stack([to_host(kv[0, h].index_select(0, ki)) for h in heads])
        kept_out = np.stack([to_host(sink[0, h]) for h in heads])
        kept_y = np.stack([to_host(y[0, h].index_select(0, ki)) for h in heads])
        gg = np.float32(to_host(g)[0])
        del c, s, sink, y
    finally:
        del kv
        _free()
    rc, rs, rg = orc.quantize(xs.reshape(-1, D), -2, 6)
    assert rg == np.float32(np.float32(8.0) / np.float32(2688.0))
    assert f"{gg!r}" == f"{rg!r}", (gg, rg)
    assert np.array_equal(ss.reshape(-1, D // 16), rs), "scales: " + first_mismatch(ss.reshape(-1, D // 16), rs)
    assert np.array_equal(cs.reshape(-1, D // 2), rc), "codes: " + first_mismatch(cs.reshape(-1, D // 2), rc)
    assert_same_floats(ys.reshape(-1, D), orc.dequantize(rc, rs, rg, "bf16"))
    assert np.array_equal(kept_out, kept_in)
    assert np.array_equal(kept_y, kept_in)


@pytest.mark.parametrize("offsets", [(0, 0), (-1, 1)], ids=["rule", "search"])
def test_mxfp4_at_the_limit(gpu, orc, offsets):
    """MXFP4 on bf16 [524288, 16384] (2^28 blocks of 32: the rule kernel's four lanes a
    block and the FP32 dequantize's 2^31 chunks at the top of their range); sampled rows
    against the oracle, codes, scales and the FP32 dequantize."""
    x = _max_tensor(torch.bfloat16, 18)
    try:
        c, s = gpu.mxfp4_quantize(x, offsets)
        y = gpu.mxfp4_dequantize(c, s, torch.float32)
        idx = _sample_rows(19).to(x.device)
        xs = to_host(x.index_select(0, idx))
        cs, ss = to_host(c.index_select(0, idx)), to_host(s.index_select(0, idx))
        ys = to_host(y.index_select(0, idx))
        del c, s, y
    finally:
        del x
        _free()
    rc, rs = orc.quantize_mxfp4(xs, *offsets)
    assert np.array_equal(ss, rs), "scales: " + first_mismatch(ss, rs)
    assert np.array_equal(cs, rc), "codes: " + first_mismatch(cs, rc)
    assert_same_floats(ys, orc.dequantize_mxfp4(rc, rs, "f32"))


def test_append_into_the_last_row_of_the_largest_cache(gpu, orc):
    """A one-token append at the device-held length 2^23 - 1 of a cache holding 2^23
    tokens per head (8 heads, 128 + 128 kept): the token leaving the recent window (ring
    slot 127) is coded into the last middle row (2^23 - 257) under the given tensor
    scale, the new token takes its ring slot, the length reaches the capacity, and a
    further append changes nothing."""
    H, D, nf, nl, capacity = 8, 128, 128, 128, 1 << 23
    print(f"[case] append at the end of a {capacity}-token cache, {H} heads", flush=True)
    cache = gpu.kv_cache_alloc(1, H, D, capacity, nf, nl)
    try:
        ring = workloads.workload(3, (1, H, nl, D))
        new = workloads.workload(4, (1, H, 1, D))
        cache["tail"].copy_(to_dev(ring))
        cache["length_dev"].fill_(capacity - 1)
        gs = torch.tensor([0.01], dtype=torch.float32, device="cuda:0")
        k_new = to_dev(new)
        gpu.kv_append_dev(cache, k_new, gs)
        length = gpu.kv_length(cache)
        last = cache["codes"].shape[2] - 1
        cs = to_host(cache["codes"][0, :, last])
        ss = to_host(cache["scales"][0, :, last])
        tail = to_host(cache["tail"])
        gpu.kv_append_dev(cache, k_new, gs)  # the cache is full: a no-op
        length2 = gpu.kv_length(cache)
        cs2, ss2 = to_host(cache["codes"][0, :, last]), to_host(cache["scales"][0, :, last])
        tail2 = to_host(cache["tail"])
    finally:
        del cache
        _free()
    assert last == capacity - nf - nl - 1
    rc, rs, _ = orc.quantize(ring[0, :, nl - 1], -2, 6, gscale=np.float32(0.01))
    assert np.array_equal(ss, rs), "scales: " + first_mismatch(ss, rs)
    assert np.array_equal(cs, rc), "codes: " + first_mismatch(cs, rc)
    want_tail = ring.copy()
    want_tail[0, :, nl - 1] = new[0, :, 0]
    assert np.array_equal(tail, want_tail)
    assert length == capacity and length2 == capacity
    assert np.array_equal(cs2, cs) and np.array_equal(ss2, ss) and np.array_equal(tail2, tail)
