"""Pins of the oracle's attention on NVFP4 operands (ScaleSearch summary page,
ScaleSearchAttention: QK^T and PV on NVFP4 operands with FP32 accumulation).

The oracle follows the readings stated in its source: operands V[code] * s with
the tensor scales applied to the products, online softmax over key tiles, P coded
per 16 keys by max scaling under S_P = fl(1/2688)."""
import numpy as np
import pytest

import ref_numpy
import workloads


def quant(orc, x, offsets=(-2, 6)):
    c, s, g = orc.quantize(x, *offsets)
    shp = x.shape[:-1]
    return c.reshape(*shp, -1), s.reshape(*shp, -1), g


def operands(orc, B, Hq, Hkv, Nq, Nk, D=128, seed=0):
    rng = np.random.default_rng(seed)
    q = workloads.to_bf16_bits(rng.standard_normal((B, Hq, Nq, D)).astype(np.float32))
    k = workloads.workload(3, (B, Hkv, Nk, D))
    v = workloads.to_bf16_bits(rng.standard_normal((B, Hkv, Nk, D)).astype(np.float32))
    return quant(orc, q), quant(orc, k), quant(orc, v)


def dequant(t):
    return ref_numpy.nvfp4_decode(t[0], t[1]) * float(t[2])


def test_uniform_scores_give_the_mean(orc):
    """Q = 0: every score is 0 and every p is 1, which codes as 6 at scale 448
    under S_P = fl(1/2688); so O is the mean of the dequantized V times
    2688 * fl(1/2688) (the tensor scale of P is a rounded reciprocal)."""
    _, k, v = operands(orc, 1, 1, 1, 8, 100)
    q = quant(orc, np.zeros((1, 1, 8, 128), np.float32))
    O, mag, bound = orc.attention_nvfp4(q, k, v)
    ref = dequant(v)[0, 0].mean(axis=0) * (2688.0 * float(np.float32(1) / np.float32(2688)))
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(ref, (8, 128)), rtol=1e-12, atol=1e-15)
    assert np.all(bound == 0)


def test_dominant_key(orc):
    """One key aligned with the query and far above the others: O = its value row."""
    D = 128
    rng = np.random.default_rng(1)
    kx = rng.standard_normal((1, 1, 64, D)).astype(np.float32) * 0.01
    kx[0, 0, 37] = 8.0
    qx = np.full((1, 1, 1, D), 8.0, np.float32)
    q, k = quant(orc, qx), quant(orc, kx)
    _, _, v = operands(orc, 1, 1, 1, 1, 64)
    O, _, _ = orc.attention_nvfp4(q, k, v)
    f = 2688.0 * float(np.float32(1) / np.float32(2688))
    np.testing.assert_allclose(O[0, 0, 0], dequant(v)[0, 0, 37] * f, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("Nq,Nk,tile,causal", [(40, 100, 32, False), (64, 64, 16, True),
                                               (33, 130, 64, False), (20, 50, 32, True)])
def test_matches_numpy_reference(orc, Nq, Nk, tile, causal):
    q, k, v = operands(orc, 1, 2, 1, Nq, Nk, seed=Nq)
    O, _, _ = orc.attention_nvfp4(q, k, v, tile=tile, causal=causal)
    ref = ref_numpy.attention_ref(q, k, v, tile=tile, causal=causal)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)


def test_causal_equals_truncated(orc):
    q, k, v = operands(orc, 1, 1, 1, 48, 48, seed=5)
    O, _, _ = orc.attention_nvfp4(q, k, v, causal=True)
    for i in (0, 15, 16, 31, 47):
        qi = tuple(a[:, :, i:i + 1] if a.ndim else a for a in q)
        ki = tuple(a[:, :, :i + 1] if a.ndim else a for a in k)
        vi = tuple(a[:, :, :i + 1] if a.ndim else a for a in v)
        Oi, _, _ = orc.attention_nvfp4(qi, ki, vi)
        np.testing.assert_array_equal(O[0, 0, i], Oi[0, 0, 0])


def test_grouped_heads(orc):
    q, k, v = operands(orc, 1, 4, 2, 24, 70, seed=7)
    O, _, _ = orc.attention_nvfp4(q, k, v)
    for h in range(4):
        sel = lambda t, hh: (t[0][:, hh:hh + 1], t[1][:, hh:hh + 1], t[2])
        Oh, _, _ = orc.attention_nvfp4(sel(q, h), sel(k, h // 2), sel(v, h // 2))
        np.testing.assert_array_equal(O[:, h:h + 1], Oh)


def test_close_to_exact_attention(orc):
    """Against FP64 softmax attention of the dequantized operands (P unquantized): the
    only difference is P's coding, a few percent of the output's scale."""
    q, k, v = operands(orc, 1, 1, 1, 64, 256, seed=9)
    O, _, _ = orc.attention_nvfp4(q, k, v)
    Q, K, V = dequant(q)[0, 0], dequant(k)[0, 0], dequant(v)[0, 0]
    S = Q @ K.T / np.sqrt(128)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    ref = (P @ V) / P.sum(axis=1, keepdims=True)
    err = np.abs(O[0, 0] - ref).max() / np.abs(ref).max()
    assert err < 0.1, err


def test_flip_allowance_is_small_and_present(orc):
    """The allowance covers only P codes near a rounding midpoint: present on some
    outputs of a realistic case, and a small part of the magnitude sum."""
    q, k, v = operands(orc, 1, 2, 1, 64, 512, seed=11)
    O, mag, bound = orc.attention_nvfp4(q, k, v)
    assert np.all(bound >= 0) and np.any(bound > 0)
    assert np.all(bound <= 0.25 * mag + 1e-300)
    assert np.median(bound / mag) < 0.02


# --- attention over the sink KV cache ---

from attn_cases import cache_of  # noqa: E402  (the sink-cache buffers the KV append builds)


@pytest.mark.parametrize("T,nf,nl", [(200, 32, 48), (90, 64, 64), (300, 0, 0), (130, 16, 0)])
def test_cache_matches_numpy_reference(orc, T, nf, nl):
    rng = np.random.default_rng(T + nf)
    qx = workloads.to_bf16_bits(rng.standard_normal((1, 2, 20, 128)).astype(np.float32))
    kx = workloads.workload(3, (1, 1, T, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, 1, T, 128)).astype(np.float32))
    q = quant(orc, qx)
    k, v = cache_of(orc, kx, nf, nl, T, T), cache_of(orc, vx, nf, nl, T, T)
    O, _, _ = orc.attention_kv_cache(q, k, v, T, nf, nl)
    ref = ref_numpy.attention_cache_ref(q, k, v, T, nf, nl)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)


def test_cache_without_sinks_is_plain_attention(orc):
    q, k, v = operands(orc, 1, 2, 1, 30, 150, seed=3)
    mk = lambda t: dict(head=np.zeros((1, 1, 0, 128), np.uint16), tail=np.zeros((1, 1, 0, 128), np.uint16),
                        codes=t[0], scales=t[1], gscale=t[2])
    O, _, _ = orc.attention_kv_cache(q, mk(k), mk(v), 150, 0, 0)
    O2, _, _ = orc.attention_nvfp4(q, k, v)
    # the two apply the tensor scales at different points in double precision
    np.testing.assert_allclose(O, O2, rtol=1e-9, atol=1e-15)


# --- split keys: units with separate softmax states, merged ---

def _cache_case(orc, T, nf, nl, Nq=3, Hq=4, Hkv=2, seed=0):
    rng = np.random.default_rng(seed)
    qx = workloads.to_bf16_bits(rng.standard_normal((1, Hq, Nq, 128)).astype(np.float32))
    kx = workloads.workload(3, (1, Hkv, T, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, Hkv, T, 128)).astype(np.float32))
    q = quant(orc, qx)
    return q, cache_of(orc, kx, nf, nl, T, T), cache_of(orc, vx, nf, nl, T, T)


@pytest.mark.parametrize("T,nf,nl,split", [(300, 32, 48, 64), (300, 32, 48, 96), (90, 64, 64, 32),
                                           (260, 0, 0, 64), (200, 16, 0, 32), (40, 64, 64, 64),
                                           (500, 128, 128, 512)])
def test_cache_split_matches_numpy_reference(orc, T, nf, nl, split):
    q, k, v = _cache_case(orc, T, nf, nl, seed=T + split)
    O, _, _ = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split)
    ref = ref_numpy.attention_cache_ref(q, k, v, T, nf, nl, split=split)
    np.testing.assert_allclose(O, ref, rtol=1e-10, atol=1e-12)


def test_cache_split_one_unit_is_the_unsplit_attention(orc):
    """No sinks and one middle piece: a single unit, whose merge weight is 1."""
    q, k, v = _cache_case(orc, 200, 0, 0, seed=5)
    O, _, _ = orc.attention_kv_cache(q, k, v, 200, 0, 0, split=256)
    O0, _, _ = orc.attention_kv_cache(q, k, v, 200, 0, 0)
    assert np.array_equal(O, O0)


def test_cache_split_is_the_mass_weighted_mean_of_unit_attentions(orc):
    """The merged output equals sum_u Z_u O_u / sum_u Z_u, where O_u is the unsplit
    oracle's attention over unit u's keys alone (as a cache of its own) and Z_u the
    softmax mass exp(s) of those keys, computed here in float64 from the decoded
    operands. Equal up to the rounding of the probabilities to binary32 in l."""
    T, nf, nl, split = 330, 32, 48, 96
    q, k, v = _cache_case(orc, T, nf, nl, Nq=2, Hq=2, Hkv=1, seed=11)
    O, _, _ = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split)
    D = 128
    qd = ref_numpy.nvfp4_decode(q[0], q[1]) * float(q[2])
    bf = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mid_hi = max(T - nl, nf)
    empty = np.zeros((1, 1, 0, D), np.uint16)

    def sub_sink(c, rows):  # bf16 rows as the head of a cache with nothing else
        return dict(head=rows, tail=empty, codes=np.zeros((1, 1, 0, D // 2), np.uint8),
                    scales=np.zeros((1, 1, 0, D // 16), np.uint8), gscale=c["gscale"])

    def sub_mid(c, a, b):
        return dict(head=empty, tail=empty, codes=c["codes"][:, :, a - nf:b - nf],
                    scales=c["scales"][:, :, a - nf:b - nf], gscale=c["gscale"])

    tail_rows = lambda c: np.stack([c["tail"][:, :, t % nl] for t in range(mid_hi, T)], axis=2)
    units = [(sub_sink(k, k["head"]), sub_sink(v, v["head"]), nf, nf,
              bf(k["head"][0, 0])),
             (sub_sink(k, tail_rows(k)), sub_sink(v, tail_rows(v)), T - mid_hi, T - mid_hi,
              bf(tail_rows(k)[0, 0]))]
    for a in range(nf, mid_hi, split):
        b = min(a + split, mid_hi)
        kd = ref_numpy.nvfp4_decode(k["codes"][0, 0, a - nf:b - nf],
                                    k["scales"][0, 0, a - nf:b - nf]) * float(k["gscale"])
        units.append((sub_mid(k, a, b), sub_mid(v, a, b), b - a, 0, kd))
    num = np.zeros_like(O)
    den = np.zeros(O.shape[:3] + (1,))
    for ku, vu, Tu, nfu, kvals in units:
        Ou, _, _ = orc.attention_kv_cache(q, ku, vu, Tu, nfu, 0)
        s = np.einsum("hqd,kd->hqk", qd[0], kvals) / np.sqrt(D)
        Z = np.exp(s - 40.0).sum(axis=-1)[None, :, :, None]
        num += Z * Ou
        den += Z
    np.testing.assert_allclose(O, num / den, rtol=1e-6, atol=1e-7 * np.abs(O).max())


def test_cache_split_must_be_whole_tiles(orc):
    q, k, v = _cache_case(orc, 100, 16, 16, seed=2)
    with pytest.raises(ValueError):
        orc.attention_kv_cache(q, k, v, 100, 16, 16, split=48)
