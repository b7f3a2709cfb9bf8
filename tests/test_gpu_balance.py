"""GPU parity of the balancing pair (ScaleSearch summary page, ScaleSearchAttention,
非干渉処理（IP）と絶対値低減: an additional pair Q' = Q R^-T, K' = K R that keeps the
scores and lowers the mean-square magnitude; reading R = diag(2^e), before the
Hadamard transform when one is used).

Bars: the calibration's exponents equal the oracle's (a channel whose a^2 / b^2 sits
within double rounding of a decision boundary may take either neighbour; none does
here); without the transform, codes, scales and tensor scale are bit-exact; with it,
the transform is within 1e-5 (relative to each vector's largest output) of the
oracle's exactly rounded one, the oracle's quantizer on the GPU's own transform
gives the GPU's bytes bit for bit, and at most 1e-4 of the blocks differ end to end."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import first_mismatch, to_dev, to_host
from test_gpu_hadamard import check_transform

pytestmark = pytest.mark.gpu

SIGNS = np.random.default_rng(21).integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)


def qk(n=1024, seed=0):
    """Q of the Q workload recipe and K of the KV workload recipe, [1, 1, n, 128] bf16."""
    return workloads.workload(5, (1, 1, n, 128)), workloads.workload(3, (1, 1, n, 128))


def gpu_exponents(nv, q, k):
    e = nv.balance_exponents(to_dev(q), to_dev(k))
    torch.cuda.synchronize()
    return e


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_calibration_matches_oracle(gpu, orc, dtype):
    q, k = qk(3000)
    if dtype == "f32":
        q, k = workloads.bf16_bits_to_f32(q) * np.float32(1.37), workloads.bf16_bits_to_f32(k)
    print(f"[case] calibration {dtype}", flush=True)
    e = to_host(gpu_exponents(gpu, q, k))
    ref = orc.balance_exponents(q, k)
    assert np.array_equal(e, ref), first_mismatch(e, ref)
    assert np.any(ref != 0)


def test_calibration_closed_form_and_degenerate(gpu, orc):
    q = np.zeros((40, 32), np.float32)
    k = np.zeros((40, 32), np.float32)
    q[:, 0], k[:, 0] = 8.0, 0.5          # e = 2
    q[:, 1], k[:, 1] = 0.5, 8.0          # e = -2
    q[:, 2], k[:, 2] = 1.0, 1.0          # balanced: 0
    q[:, 3] = 1.0                        # K channel zero: 0
    e = to_host(gpu_exponents(gpu, q, k))
    assert list(e[:4]) == [2, -2, 0, 0] and np.all(e[4:] == 0)
    np.testing.assert_array_equal(e, orc.balance_exponents(q, k))
    # no rows at all: every exponent 0
    e0 = to_host(gpu_exponents(gpu, q[:0], k[:0]))
    assert np.all(e0 == 0)


def quantize_case(nv, orc, x, e, side, offsets, hadamard=False, signs=None):
    print(f"[case] balanced quantize {x.shape} {x.dtype} side={side} offsets={offsets} "
          f"hadamard={hadamard} signs={signs is not None}", flush=True)
    ed = torch.from_numpy(np.ascontiguousarray(e)).cuda()
    xd = to_dev(x)
    bal = (ed, "q" if side < 0 else "k")
    c, s, g = nv.quantize(xd, offsets, hadamard=hadamard, signs=signs, balance=bal)
    torch.cuda.synchronize()
    gc, gs, gg = to_host(c), to_host(s), np.float32(to_host(g)[0])
    K = x.shape[-1]
    if not hadamard:
        rc, rs, rg = orc.quantize_balanced(x, e, side, *offsets)
        assert gg == rg or (np.isnan(gg) and np.isnan(rg))
        assert np.array_equal(gs.reshape(rs.shape), rs), "scales: " + first_mismatch(gs, rs)
        assert np.array_equal(gc.reshape(rc.shape), rc), "codes: " + first_mismatch(gc, rc)
        return
    y = to_host(nv.hadamard128(xd, signs=signs, balance=bal)).reshape(-1, K)
    ref = orc.hadamard128_balanced(x.reshape(-1, K), e, side, signs)
    exact, nae = check_transform(y, ref)
    # split parity: the oracle's quantizer on the GPU's own transform
    rc, rs, rg = orc.quantize(y, *offsets)
    assert gg == rg
    assert np.array_equal(gs.reshape(rs.shape), rs), "scales: " + first_mismatch(gs, rs)
    assert np.array_equal(gc.reshape(rc.shape), rc), "codes: " + first_mismatch(gc, rc)
    ec, es, eg = orc.quantize_balanced(x, e, side, *offsets, hadamard=True, signs=signs)
    bad = (es.reshape(-1) != gs.reshape(-1)) | np.any(ec.reshape(-1, 8) != gc.reshape(-1, 8), axis=1)
    print(f"[balance] transform {exact:.4f} bit-exact, NAE {nae:.2e}; {bad.sum()} of {bad.size} "
          f"blocks differ end to end", flush=True)
    assert bad.mean() <= 1e-4


@pytest.mark.parametrize("offsets", [(-2, 6), (-8, 8), (0, 0), (-3, 4)])
@pytest.mark.parametrize("side", [-1, 1])
def test_quantize_without_transform(gpu, orc, offsets, side):
    q, k = qk(600)
    e = orc.balance_exponents(q, k)
    x = q if side < 0 else k
    quantize_case(gpu, orc, x.reshape(-1, 128), e, side, offsets)


def test_quantize_fp32_wide_rows_and_edges(gpu, orc):
    """FP32 rows of 48 blocks with exponents across [-32, 32] (clamped beyond) and
    values pushed into the subnormal range and to overflow (Inf: the non-finite
    contract) by their channel's factor."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((37, 768)) * np.exp(rng.normal(0, 3, (1, 768)))).astype(np.float32)
    e = rng.integers(-40, 41, 768).astype(np.int8)
    quantize_case(gpu, orc, x, e, 1, (-2, 6))
    x2 = x.copy()
    x2[:, 5] = 1e-30
    e2 = np.zeros(768, np.int8)
    e2[5] = -32                              # 1e-30 * 2^-32: subnormal in binary32
    quantize_case(gpu, orc, x2, e2, 1, (-8, 8))
    e3 = np.zeros(768, np.int8)
    e3[7] = 32
    x3 = x.copy()
    x3[3, 7] = 3e38                          # overflows to Inf: S_g NaN
    quantize_case(gpu, orc, x3, e3, 1, (-2, 6))


def test_zero_exponents_are_the_plain_quantizer(gpu, orc):
    x = workloads.workload(4, (64, 512))
    xd = to_dev(x)
    z = torch.zeros(512, dtype=torch.int8, device="cuda:0")
    c, s, g = gpu.quantize(xd, (-2, 6), balance=(z, "k"))
    c0, s0, g0 = gpu.quantize(xd, (-2, 6))
    torch.cuda.synchronize()
    assert torch.equal(c, c0) and torch.equal(s, s0) and torch.equal(g, g0)


@pytest.mark.parametrize("signs", [None, SIGNS])
@pytest.mark.parametrize("side", [-1, 1])
def test_quantize_with_transform(gpu, orc, signs, side):
    q, k = qk(1500)
    e = orc.balance_exponents(q, k)
    x = q if side < 0 else k
    quantize_case(gpu, orc, x, e, side, (-8, 8) if side < 0 else (-2, 6), hadamard=True,
                  signs=signs)


def test_scores_kept_through_the_transform(gpu, orc):
    """(Q 2^-e H_s)(K 2^e H_s)^T against QK^T in double: FP32 transform rounding only."""
    q, k = qk(256)
    e = orc.balance_exponents(q, k)
    ed = torch.from_numpy(e).cuda()
    yq = to_host(gpu.hadamard128(to_dev(q), signs=SIGNS, balance=(ed, "q"))).reshape(-1, 128)
    yk = to_host(gpu.hadamard128(to_dev(k), signs=SIGNS, balance=(ed, "k"))).reshape(-1, 128)
    Q = workloads.bf16_bits_to_f32(q).reshape(-1, 128).astype(np.float64)
    K = workloads.bf16_bits_to_f32(k).reshape(-1, 128).astype(np.float64)
    S = Q @ K.T
    err = np.abs(yq.astype(np.float64) @ yk.astype(np.float64).T - S)
    assert np.all(err <= 1e-5 * (np.abs(Q) @ np.abs(K).T))


def test_full_size(gpu, orc):
    """Workload 5's Q [1, 32, 32768, 128] with the randomized transform and offsets
    [-8, 8], balanced against workload 3's K recipe [1, 8, 32768, 128]: exponents
    from the calibration of the two, the Q side quantized at full size; the
    transform checked in chunks of four heads."""
    q = workloads.workload(5)
    k = workloads.workload(3)
    e = orc.balance_exponents(q, k)
    eg = to_host(gpu_exponents(gpu, q, k))
    assert np.array_equal(eg, e), first_mismatch(eg, e)
    print("[case] balanced full size", flush=True)
    ed = torch.from_numpy(e).cuda()
    qd = to_dev(q)
    c, s, g = gpu.quantize(qd, (-8, 8), signs=SIGNS, balance=(ed, "q"))
    torch.cuda.synchronize()
    gc, gs, gg = to_host(c), to_host(s), np.float32(to_host(g)[0])
    ec, es, egs = orc.quantize_balanced(q, e, -1, -8, 8, hadamard=True, signs=SIGNS)
    assert abs(float(gg) - float(egs)) <= 1e-5 * float(egs)
    bad = (es.reshape(-1) != gs.reshape(-1)) | np.any(ec.reshape(-1, 8) != gc.reshape(-1, 8), axis=1)
    print(f"[balance] full size: {bad.sum()} of {bad.size} blocks differ end to end", flush=True)
    assert bad.mean() <= 1e-4
    for h0 in range(0, 32, 4):
        part = np.ascontiguousarray(q[:, h0:h0 + 4]).reshape(-1, 128)
        y = to_host(gpu.hadamard128(qd[:, h0:h0 + 4].contiguous(), signs=SIGNS,
                                    balance=(ed, "q"))).reshape(-1, 128)
        check_transform(y, orc.hadamard128_balanced(part, e, -1, SIGNS))
