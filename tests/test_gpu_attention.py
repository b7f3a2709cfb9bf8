"""GPU parity of attention on NVFP4 operands (ScaleSearch summary page,
ScaleSearchAttention: QK^T and PV with NVFP4 operands and FP32 accumulation).

The operands are coded by the oracle (so no input comes from the HIP path) and
uploaded. The kernel's products are exact but its sums run in FP32 in the
matrix units' order, and its P codes come from binary32 scores and exp, so the
bar is a per-element bound derived from that arithmetic (u = 2^-24):

  |O_gpu - O| <= mag * (Nk + 8 * tiles + 64) u        (FP32 sums of P^ v, rescales)
               + |O| * (delta + (Nk + 64) u)          (the softmax sum l)
               + bound                                (P codes that may round the other way)

with O, mag and bound from the oracle and delta the relative error the scores
and exp can put on a p (the oracle's own allowance formula)."""
import numpy as np
import pytest
import torch

import ref_numpy
import ref_numpy as R
import workloads
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def coded(orc, x):
    c, s, g = orc.quantize(x, -2, 6)
    shp = x.shape[:-1]
    return c.reshape(*shp, 64), s.reshape(*shp, 8), g


def make_ops(orc, B, Hq, Hkv, Nq, Nk, seed):
    rng = np.random.default_rng(seed)
    q = workloads.to_bf16_bits(rng.standard_normal((B, Hq, Nq, 128)).astype(np.float32))
    k = workloads.workload(3, (B, Hkv, Nk, 128))
    v = workloads.to_bf16_bits(rng.standard_normal((B, Hkv, Nk, 128)).astype(np.float32))
    return coded(orc, q), coded(orc, k), coded(orc, v)


def upload(t):
    c, s, g = t
    return (torch.from_numpy(np.ascontiguousarray(c)).cuda(),
            torch.from_numpy(np.ascontiguousarray(s)).cuda(),
            torch.tensor([g], dtype=torch.float32, device="cuda:0"))


def score_delta(q, k):
    """Largest relative error binary32 scores and exp can put on a p (the oracle's formula)."""
    Q = ref_numpy.nvfp4_decode(q[0], q[1])
    K = ref_numpy.nvfp4_decode(k[0], k[1])
    c = float(q[2]) * float(k[2]) / np.sqrt(128.0)
    Hq, Hkv = Q.shape[1], K.shape[1]
    worst = 0.0
    for h in range(Hq):
        Qh, Kh = Q[:, h], K[:, h // (Hq // Hkv)]
        A = np.einsum("bid,bjd->bij", np.abs(Qh), np.abs(Kh)) * c
        S = np.einsum("bid,bjd->bij", Qh, Kh) * c
        worst = max(worst, float(A.max(initial=0.0)) * 130 * U + 2 * float(np.abs(S).max(initial=0.0))
                    * 2.0 ** -21 + 2.0 ** -20)
    return worst


def check(gpu, orc, q, k, v, causal=False, out_dtype=torch.float32):
    Nk = k[0].shape[2]
    print(f"[case] attention q={q[0].shape} k={k[0].shape} causal={causal} out={out_dtype}",
          flush=True)
    O = gpu.attention(upload(q), upload(k), upload(v), causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = to_host(O.float()).astype(np.float64)
    ref, mag, bound = orc.attention_nvfp4(q, k, v, tile=32, causal=causal)
    tiles = -(-Nk // 32)
    delta = score_delta(q, k)
    tol = mag * (Nk + 8 * tiles + 64) * U + np.abs(ref) * (delta + (Nk + 64) * U) + bound
    if out_dtype == torch.bfloat16:
        tol = tol + np.abs(ref) * 2.0 ** -8
    err = np.abs(got - ref)
    ratio = float(np.max(err / np.maximum(tol, 1e-300)))
    print(f"[attention] max err/tol {ratio:.3f}, max err {err.max():.3e}, "
          f"elements with a flip allowance {np.mean(bound > 0):.4f}")
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements outside the bound; first at {np.argwhere(bad)[0]}"
    return got, ref


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", [(1, 2, 1, 300, 1000), (2, 1, 1, 128, 32),
                                             (1, 4, 2, 77, 513), (1, 1, 1, 1, 5)])
def test_parity(gpu, orc, B, Hq, Hkv, Nq, Nk):
    check(gpu, orc, *make_ops(orc, B, Hq, Hkv, Nq, Nk, seed=Nq + Nk))


@pytest.mark.parametrize("Nq,Nk", [(257, 257), (100, 300), (300, 100)])
def test_causal(gpu, orc, Nq, Nk):
    check(gpu, orc, *make_ops(orc, 1, 2, 2, Nq, Nk, seed=Nq * 3 + Nk), causal=True)


def test_bf16_output(gpu, orc):
    check(gpu, orc, *make_ops(orc, 1, 1, 1, 200, 400, seed=3), out_dtype=torch.bfloat16)


def test_hadamard_operands(gpu, orc):
    """Q and K coded after the same randomized Hadamard transform (their product is
    unchanged): the attention of the transformed operands, same bar."""
    rng = np.random.default_rng(8)
    signs = rng.integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)
    qx = workloads.workload(5, (1, 4, 200, 128))
    kx = workloads.workload(3, (1, 1, 700, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, 1, 700, 128)).astype(np.float32))

    def rht(x):
        c, s, g = orc.quantize_rht(x, signs, -8, 8)
        return c.reshape(*x.shape[:-1], 64), s.reshape(*x.shape[:-1], 8), g

    check(gpu, orc, rht(qx), rht(kx), coded(orc, vx))


def test_no_keys_and_no_queries(gpu, orc):
    q, k, v = make_ops(orc, 1, 1, 1, 40, 0, seed=1)
    O = gpu.attention(upload(q), upload(k), upload(v))
    torch.cuda.synchronize()
    assert torch.all(O == 0)
    q, k, v = make_ops(orc, 1, 1, 1, 0, 64, seed=2)
    O = gpu.attention(upload(q), upload(k), upload(v))
    assert O.shape == (1, 1, 0, 128)


def test_full_size_sampled_rows(gpu, orc):
    """Q [1, 32, 32768, 128] against K, V [1, 8, 32768, 128] (grouped heads), non-causal,
    the benchmark's launch; the oracle evaluates 4 sampled query rows of every head."""
    rng = np.random.default_rng(17)
    qx = workloads.workload(5)
    kx = workloads.workload(3)
    vx = workloads.to_bf16_bits(rng.standard_normal(kx.shape).astype(np.float32))
    q, k, v = coded(orc, qx), coded(orc, kx), coded(orc, vx)
    O = gpu.attention(upload(q), upload(k), upload(v))
    torch.cuda.synchronize()
    got_all = to_host(O)
    rows = np.sort(rng.choice(32768, 4, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 32767]]))
    qs = (q[0][:, :, rows], q[1][:, :, rows], q[2])
    ref, mag, bound = orc.attention_nvfp4(qs, k, v)
    got = got_all[:, :, rows].astype(np.float64)
    Nk = 32768
    delta = score_delta(qs, k)
    tol = mag * (Nk + 8 * 1024 + 64) * U + np.abs(ref) * (delta + (Nk + 64) * U) + bound
    err = np.abs(got - ref)
    print(f"[attention] full size: max err/tol {float(np.max(err / tol)):.3f}")
    assert np.all(err <= tol)


# --- attention over the sink KV cache (the cache is built by the oracle) ---

def upload_cache(c, T, nf, nl):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: t(a.view(np.int16)).view(torch.bfloat16)
    return dict(head=bf(c["head"]), tail=bf(c["tail"]), codes=t(c["codes"]), scales=t(c["scales"]),
                n_first=nf, n_last=nl, length=T), \
        torch.tensor([c["gscale"]], dtype=torch.float32, device="cuda:0")


def cache_case(orc, Hq, Hkv, Nq, T, nf, nl, seed):
    """Q coded by the oracle and K, V sink caches built by the oracle (cap = middle + 8)."""
    from test_oracle_attention import cache_of

    rng = np.random.default_rng(seed)
    qx = workloads.to_bf16_bits(rng.standard_normal((1, Hq, Nq, 128)).astype(np.float32))
    kx = workloads.workload(3, (1, Hkv, T, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, Hkv, T, 128)).astype(np.float32))
    q = coded(orc, qx)
    cap = max(T - nf - nl, 0) + 8
    return q, cache_of(orc, kx, nf, nl, T, cap), cache_of(orc, vx, nf, nl, T, cap)


def cache_tol(q, k, T, nf, nl, ref, mag, bound, units=1):
    """The bound of the module docstring over the cache's T keys; with split keys,
    plus the merge: units weights 2^(m_u - M) in binary32 (a few u each) and the
    FP32 sums over the units, on the numerator (mag) and on l (|O|)."""
    Hq, Hkv = q[0].shape[1], k["codes"].shape[1]
    tiles = -(-T // 32) + 3
    Qd = R.nvfp4_decode(q[0], q[1]) * float(q[2])
    Kd = R.cache_values(k, T, nf, nl)
    delta = 0.0
    for h in range(Hq):
        Kh = Kd[:, h // (Hq // Hkv)]
        A = np.einsum("bid,bjd->bij", np.abs(Qd[:, h]), np.abs(Kh)) / np.sqrt(128.0)
        S = np.einsum("bid,bjd->bij", Qd[:, h], Kh) / np.sqrt(128.0)
        delta = max(delta, float(A.max(initial=0.0)) * 130 * U +
                    2 * float(np.abs(S).max(initial=0.0)) * 2.0 ** -21 + 2.0 ** -20)
    merge = (units + 16) * U if units > 1 else 0.0
    return (mag * ((T + 8 * tiles + 64) * U + merge) +
            np.abs(ref) * (delta + (T + 64) * U + merge) + bound)


@pytest.mark.parametrize("Hq,Hkv,Nq,T,nf,nl", [(2, 1, 77, 1000, 128, 128), (4, 2, 40, 300, 64, 0),
                                                (1, 1, 33, 90, 64, 64), (1, 1, 20, 50, 64, 16),
                                                (2, 2, 64, 200, 0, 0), (1, 1, 5, 520, 32, 96),
                                                (8, 1, 17, 300, 16, 16)])
def test_kv_cache_attention(gpu, orc, Hq, Hkv, Nq, T, nf, nl):
    q, k, v = cache_case(orc, Hq, Hkv, Nq, T, nf, nl, T + 7 * nf + nl)
    print(f"[case] kv-cache attention Hq={Hq} Hkv={Hkv} Nq={Nq} T={T} nf={nf} nl={nl}", flush=True)
    kc, kg = upload_cache(k, T, nf, nl)
    vc, vg = upload_cache(v, T, nf, nl)
    O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg)
    torch.cuda.synchronize()
    got = to_host(O).astype(np.float64)
    ref, mag, bound = orc.attention_kv_cache(q, k, v, T, nf, nl)
    tol = cache_tol(q, k, T, nf, nl, ref, mag, bound)
    err = np.abs(got - ref)
    print(f"[attention] kv cache: max err/tol {float(np.max(err / np.maximum(tol, 1e-300))):.3f}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("Hq,Hkv,Nq,T,nf,nl,split", [
    (32, 8, 1, 3000, 128, 128, 256),   # decode, grouped heads, a short last piece
    (4, 2, 40, 300, 64, 0, 64),
    (1, 1, 5, 520, 32, 96, 96),        # pieces of one and a half chunks
    (2, 1, 3, 50, 64, 16, 32),         # fewer tokens than the head: empty middle and tail
    (2, 2, 1, 200, 0, 0, 32),          # no sinks: empty head and tail units
    (8, 1, 16, 700, 16, 16, 128),      # 8 heads x 16 queries: one full workgroup
    (8, 1, 17, 700, 16, 16, 128),      # 136 rows: a second workgroup across two heads
])
def test_kv_cache_attention_split(gpu, orc, Hq, Hkv, Nq, T, nf, nl, split):
    q, k, v = cache_case(orc, Hq, Hkv, Nq, T, nf, nl, T + split + Nq)
    print(f"[case] split kv-cache attention Hq={Hq} Hkv={Hkv} Nq={Nq} T={T} nf={nf} nl={nl} "
          f"split={split}", flush=True)
    kc, kg = upload_cache(k, T, nf, nl)
    vc, vg = upload_cache(v, T, nf, nl)
    cap = kc["codes"].shape[2]
    units = 2 + -(-cap // split)
    ws = torch.full((gpu.attention_split_workspace_bytes(1, Hq, Nq, cap, split),), 0xFF,
                    dtype=torch.uint8, device="cuda:0")   # NaN patterns: every read slot is written
    for dt in (torch.float32, torch.bfloat16):
        O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg, out_dtype=dt, split=split,
                                   workspace=ws)
        torch.cuda.synchronize()
        got = to_host(O.float()).astype(np.float64)
        ref, mag, bound = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split)
        tol = cache_tol(q, k, T, nf, nl, ref, mag, bound, units)
        if dt == torch.bfloat16:
            tol = tol + np.abs(ref) * 2.0 ** -8
        err = np.abs(got - ref)
        print(f"[attention] split kv cache {dt}: max err/tol "
              f"{float(np.max(err / np.maximum(tol, 1e-300))):.3f}")
        assert np.all(err <= tol)


@pytest.mark.parametrize("split", [160, 512])
def test_kv_cache_attention_split_full_size_decode(gpu, orc, split):
    """One decode query per head, Hq = 32 over Hkv = 8, a cache of 128 + 32768 + 128
    tokens, split into pieces of 160 (the benchmark's decode step) and of 512: every
    row against the oracle."""
    Hq, Hkv, Nq, nf, nl = 32, 8, 1, 128, 128
    T = nf + 32768 + nl
    q, k, v = cache_case(orc, Hq, Hkv, Nq, T, nf, nl, 2024)
    print(f"[case] split kv-cache attention, full-size decode, pieces of {split}", flush=True)
    kc, kg = upload_cache(k, T, nf, nl)
    vc, vg = upload_cache(v, T, nf, nl)
    cap = kc["codes"].shape[2]
    O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg, split=split)
    torch.cuda.synchronize()
    got = to_host(O).astype(np.float64)
    ref, mag, bound = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split)
    tol = cache_tol(q, k, T, nf, nl, ref, mag, bound, 2 + -(-cap // split))
    err = np.abs(got - ref)
    print(f"[attention] full-size decode: max err/tol {float(np.max(err / tol)):.3f}")
    assert np.all(err <= tol)


def test_kv_cache_attention_empty_cache(gpu, orc):
    """A cache that holds no token: every unit of the split call is empty (its state
    max -inf, sum 0) and the output is 0, as the unsplit call and the oracle give; the
    same through the device-held length."""
    q = coded(orc, workloads.to_bf16_bits(
        np.random.default_rng(9).standard_normal((1, 4, 3, 128)).astype(np.float32)))
    empty = dict(head=np.zeros((1, 2, 16, 128), np.uint16), tail=np.zeros((1, 2, 16, 128), np.uint16),
                 codes=np.zeros((1, 2, 64, 64), np.uint8), scales=np.zeros((1, 2, 64, 8), np.uint8),
                 gscale=np.float32(1))
    ref, _, _ = orc.attention_kv_cache(q, empty, empty, 0, 16, 16, split=32)
    assert np.all(ref == 0)
    kc, g = upload_cache(empty, 0, 16, 16)
    kc["length_dev"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    qd = upload(q)
    for kw in (dict(), dict(split=32), dict(split=32, device_length=True),
               dict(device_length=True)):
        print(f"[case] empty cache {kw}", flush=True)
        O = gpu.attention_kv_cache(qd, kc, g, kc, g, **kw)
        torch.cuda.synchronize()
        assert O.shape == (1, 4, 3, 128) and torch.all(O == 0), kw
