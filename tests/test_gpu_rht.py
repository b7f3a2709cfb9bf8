"""GPU checks of the randomized Hadamard transform (random +-1 signs before the
128-point transform, QuIP#-style incoherence processing; ScaleSearch summary
page, ScaleSearchAttention, 非干渉処理（IP）と絶対値低減: a transform pair Q' = Q R^-T,
K' = K R that keeps Q K^T).

Same bars as the plain transform (the MFMA accumulates in FP32): the transform
within 1e-5 of the oracle's exactly rounded one, split parity bit for bit, and
at most 1e-4 of the blocks differing end to end. The sign flip itself is exact,
so the randomized transform of x must equal the plain transform of x o s bit
for bit on the GPU.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import first_mismatch, to_dev, to_host
from test_gpu_hadamard import check_transform

pytestmark = pytest.mark.gpu


def draw_signs(seed):
    return np.random.default_rng(seed).integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)


def flip(x_bits, signs):
    """x o s on bf16 bit patterns: toggle the sign bit of the features whose bit is set."""
    bits = np.array([(int(signs[k // 32]) >> (k % 32)) & 1 for k in range(128)], np.uint16)
    shp = x_bits.shape
    return (x_bits.reshape(-1, 128) ^ (bits << 15)).reshape(shp)


@pytest.mark.parametrize("shape,seed", [((1, 2, 333, 128), 11), ((5, 256), 12),
                                        ((3, 1024), 13)])
def test_transform(gpu, orc, shape, seed):
    x = workloads.workload(5, shape)
    s = draw_signs(seed)
    xd = to_dev(x)
    y = to_host(gpu.hadamard128(xd, signs=s))
    exact, nae = check_transform(y, orc.hadamard128_rht(x, s))
    print(f"[rht] {shape}: {exact:.4f} of outputs bit-exact, NAE {nae:.2e}")
    # the sign flip is exact: same bits as the plain transform of x o s
    yp = to_host(gpu.hadamard128(to_dev(flip(x, s))))
    np.testing.assert_array_equal(y.view(np.uint32), yp.view(np.uint32))


def test_zero_signs_are_the_plain_transform(gpu):
    x = workloads.workload(5, (1, 1, 100, 128))
    xd = to_dev(x)
    z = np.zeros(4, np.uint32)
    np.testing.assert_array_equal(to_host(gpu.hadamard128(xd, signs=z)).view(np.uint32),
                                  to_host(gpu.hadamard128(xd)).view(np.uint32))
    c0, s0, g0 = gpu.quantize(xd, (-8, 8), signs=z)
    c1, s1, g1 = gpu.quantize(xd, (-8, 8), hadamard=True)
    torch.cuda.synchronize()
    assert g0.item() == g1.item()
    assert torch.equal(c0, c1) and torch.equal(s0, s1)


def _split_and_end_to_end(gpu, orc, x, s, offsets=(-8, 8)):
    xd = to_dev(x)
    c, sc, g = gpu.quantize(xd, offsets, signs=s)
    y = gpu.hadamard128(xd, signs=s)
    torch.cuda.synchronize()
    gc, gs, gg = to_host(c), to_host(sc), np.float32(to_host(g)[0])
    yh = to_host(y).reshape(-1, x.shape[-1])
    rc, rs, rg = orc.quantize(yh, *offsets)
    assert gg == rg
    assert np.array_equal(gs.reshape(rs.shape), rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc.reshape(rc.shape), rc), "codes: " + first_mismatch(gc, rc)
    ec, es, eg = orc.quantize_rht(x.reshape(-1, x.shape[-1]), s, *offsets)
    assert abs(float(gg) - float(eg)) <= 1e-5 * float(eg)
    bad = (es != gs.reshape(es.shape)) | np.any(
        ec.reshape(-1, 8) != gc.reshape(-1, 8), axis=1).reshape(es.shape)
    print(f"[rht] {x.shape}: {bad.sum()} of {bad.size} blocks differ end to end "
          f"({bad.mean():.2e})")
    assert bad.mean() <= 1e-4


@pytest.mark.parametrize("shape", [(1, 4, 2048, 128), (7, 384), (1, 1, 33, 128)])
def test_quantize_rht_shrunk(gpu, orc, shape):
    _split_and_end_to_end(gpu, orc, workloads.workload(5, shape), draw_signs(21))


def test_quantize_rht_full(gpu, orc):
    """Workload 5 at full size: bf16 Q [1, 32, 32768, 128], offsets [-8, 8]."""
    _split_and_end_to_end(gpu, orc, workloads.workload(5), draw_signs(22))


def test_global_scale_rht(gpu, orc):
    x = workloads.workload(5, (1, 2, 500, 128))
    s = draw_signs(23)
    xd = to_dev(x)
    g = gpu.global_scale(xd, signs=s)
    y = gpu.hadamard128(xd, signs=s)
    torch.cuda.synchronize()
    _, _, rg = orc.quantize(to_host(y).reshape(-1, 128), 0, 0)
    assert np.float32(g.item()) == rg


def test_sink_mode_rht(gpu, orc):
    kv = workloads.workload(3, (1, 3, 700, 128))
    s = draw_signs(24)
    kvd = to_dev(kv)
    c, sc, g, sink = gpu.quantize_kv_sink(kvd, 128, 128, (-8, 8), signs=s)
    torch.cuda.synchronize()
    # the sink tokens stay in full precision, untransformed
    assert np.array_equal(to_host(sink)[:, :, :128], kv[:, :, :128])
    assert np.array_equal(to_host(sink)[:, :, 128:], kv[:, :, 700 - 128:])
    mid = kvd[:, :, 128:700 - 128].contiguous()
    y = to_host(gpu.hadamard128(mid, signs=s)).reshape(-1, 128)
    rc, rs, rg = orc.quantize(y, -8, 8)
    assert np.float32(to_host(g)[0]) == rg
    assert np.array_equal(to_host(sc).reshape(rs.shape), rs)
    assert np.array_equal(to_host(c).reshape(rc.shape), rc)


def test_append_rht_matches_one_shot(gpu):
    """Appending in pieces gives what the one-shot sink mode gives (same kernels, so
    bit for bit), with the randomized transform on the coded tokens."""
    B, H, D, nf, nl = 1, 2, 128, 32, 48
    steps = [150, 1, 1, 40, 1, 7]
    total = sum(steps)
    kv_all = workloads.workload(3, (B, H, total, D))
    s = draw_signs(25)
    sg = np.float32(np.abs(workloads.bf16_bits_to_f32(kv_all[:, :, :150])).max() / 2688.0)
    g = torch.tensor([sg], dtype=torch.float32, device="cuda:0")
    cache = gpu.kv_cache_alloc(B, H, D, capacity=total, n_first=nf, n_last=nl)
    t = 0
    for k in steps:
        print(f"[case] rht append {k} tokens at {t}", flush=True)
        gpu.kv_append(cache, to_dev(np.ascontiguousarray(kv_all[:, :, t:t + k])), g, (-8, 8),
                      signs=s)
        t += k
        rc, rs, _, rsink = gpu.quantize_kv_sink(to_dev(np.ascontiguousarray(kv_all[:, :, :t])),
                                                nf, nl, (-8, 8), global_scale=g, signs=s)
        torch.cuda.synchronize()
        tm = t - nf - nl
        assert torch.equal(cache["codes"][:, :, :tm], rc)
        assert torch.equal(cache["scales"][:, :, :tm], rs)
        assert torch.equal(cache["head"], rsink[:, :, :nf])


def test_scores_preserved(gpu):
    """(Q R)(K R)^T = Q K^T with R = diag(s) H / sqrt(128) orthogonal: the GPU's
    transformed Q and K give the same scores to FP32 accuracy."""
    q = workloads.workload(5, (1, 1, 256, 128))
    k = workloads.workload(3, (1, 1, 256, 128))
    s = draw_signs(26)
    qt = gpu.hadamard128(to_dev(q), signs=s).double().reshape(256, 128)
    kt = gpu.hadamard128(to_dev(k), signs=s).double().reshape(256, 128)
    qf = torch.from_numpy(workloads.bf16_bits_to_f32(q).reshape(256, 128)).double()
    kf = torch.from_numpy(workloads.bf16_bits_to_f32(k).reshape(256, 128)).double()
    ref = qf @ kf.T
    got = (qt @ kt.T).cpu()
    scale = (qf.abs() @ kf.abs().T)
    assert torch.all((got - ref).abs() <= 1e-5 * scale + 1e-30)
