"""GPU parity of attention on NVFP4 operands (ScaleSearch summary page,
ScaleSearchAttention, ネイティブ NVFP4 実行: QK^T and PV with NVFP4 operands and FP32
accumulation).

The operands are coded by the oracle (so no input comes from the HIP path) and
uploaded. The kernel's products are exact but its sums run in FP32 in the matrix
units' order, and its P codes come from binary32 scores and exp, so the bar is the
per-element bound of tests/attn_tol.py, built from the oracle's terms (FP32 sums of
P^ v tile by tile, the rescales and merge weights, P coded against an earlier running
max, the softmax sum l, and P codes that may round the other way). The CPU tests in
tests/test_attention_bar.py check that bar at these same shapes from both sides: a
binary32 emulation stays inside it, and a dropped key, a dropped 16-key block of
P^ v, a P code one step off or 64-key tiles leave it."""
import numpy as np
import pytest
import torch

import attn_cases as AC
import workloads
import attn_tol as T_
from gpu_util import to_host

pytestmark = pytest.mark.gpu

coded, make_ops, cache_of = AC.coded, AC.make_ops, AC.cache_of


def upload(t):
    c, s, g = t
    return (torch.from_numpy(np.ascontiguousarray(c)).cuda(),
            torch.from_numpy(np.ascontiguousarray(s)).cuda(),
            torch.tensor([g], dtype=torch.float32, device="cuda:0"))


def within(got, ref, tol, what):
    err = np.abs(got - ref)
    ratio = float(np.max(err / np.maximum(tol, 1e-300), initial=0.0))
    print(f"[attention] {what}: max err/bar {ratio:.3f}, max err {err.max(initial=0):.3e}", flush=True)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements outside the bar; first at {np.argwhere(bad)[0]}"


def check(gpu, orc, q, k, v, causal=False, out_dtype=torch.float32):
    print(f"[case] attention q={q[0].shape} k={k[0].shape} causal={causal} out={out_dtype}",
          flush=True)
    O = gpu.attention(upload(q), upload(k), upload(v), causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = to_host(O.float()).astype(np.float64)
    ref, mag, bound, terms = orc.attention_nvfp4(q, k, v, tile=32, causal=causal, terms=True)
    tol = T_.attention_tol(ref, mag, bound, terms, out_bf16=out_dtype == torch.bfloat16)
    within(got, ref, tol, f"q={q[0].shape} causal={causal}")
    return got, ref


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", AC.PREFILL_SHAPES)
def test_parity(gpu, orc, B, Hq, Hkv, Nq, Nk):
    check(gpu, orc, *make_ops(orc, B, Hq, Hkv, Nq, Nk, seed=Nq + Nk))


@pytest.mark.parametrize("Nq,Nk", AC.CAUSAL_SHAPES)
def test_causal(gpu, orc, Nq, Nk):
    check(gpu, orc, *make_ops(orc, 1, 2, 2, Nq, Nk, seed=Nq * 3 + Nk), causal=True)


def test_bf16_output(gpu, orc):
    check(gpu, orc, *make_ops(orc, 1, 1, 1, 200, 400, seed=3), out_dtype=torch.bfloat16)


def test_hadamard_operands(gpu, orc):
    """Q and K coded after the same randomized Hadamard transform (their product is
    unchanged): the attention of the transformed operands, same bar."""
    check(gpu, orc, *AC.hadamard_ops(orc))


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
    the benchmark's launch; the oracle evaluates the sampled query rows of every head."""
    q, k, v = AC.full_size_ops(orc)
    print("[case] attention full size", flush=True)
    O = gpu.attention(upload(q), upload(k), upload(v))
    torch.cuda.synchronize()
    rows = AC.sampled_rows()
    got = to_host(O)[:, :, rows].astype(np.float64)
    qs = (q[0][:, :, rows], q[1][:, :, rows], q[2])
    ref, mag, bound, terms = orc.attention_nvfp4(qs, k, v, terms=True)
    within(got, ref, T_.attention_tol(ref, mag, bound, terms), "full size")


# --- attention over the sink KV cache (the cache is built by the oracle) ---

def upload_cache(c, T, nf, nl):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: t(a.view(np.int16)).view(torch.bfloat16)
    return dict(head=bf(c["head"]), tail=bf(c["tail"]), codes=t(c["codes"]), scales=t(c["scales"]),
                n_first=nf, n_last=nl, length=T), \
        torch.tensor([c["gscale"]], dtype=torch.float32, device="cuda:0")


cache_case = AC.cache_case


@pytest.mark.parametrize("Hq,Hkv,Nq,T,nf,nl", AC.CACHE_SHAPES)
def test_kv_cache_attention(gpu, orc, Hq, Hkv, Nq, T, nf, nl):
    q, k, v = cache_case(orc, Hq, Hkv, Nq, T, nf, nl, T + 7 * nf + nl)
    print(f"[case] kv-cache attention Hq={Hq} Hkv={Hkv} Nq={Nq} T={T} nf={nf} nl={nl}", flush=True)
    kc, kg = upload_cache(k, T, nf, nl)
    vc, vg = upload_cache(v, T, nf, nl)
    O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg)
    torch.cuda.synchronize()
    got = to_host(O).astype(np.float64)
    ref, mag, bound, terms = orc.attention_kv_cache(q, k, v, T, nf, nl, terms=True)
    within(got, ref, T_.attention_tol(ref, mag, bound, terms), "kv cache")


@pytest.mark.parametrize("Hq,Hkv,Nq,T,nf,nl,split", AC.SPLIT_SHAPES)
def test_kv_cache_attention_split(gpu, orc, Hq, Hkv, Nq, T, nf, nl, split):
    q, k, v = cache_case(orc, Hq, Hkv, Nq, T, nf, nl, T + split + Nq)
    print(f"[case] split kv-cache attention Hq={Hq} Hkv={Hkv} Nq={Nq} T={T} nf={nf} nl={nl} "
          f"split={split}", flush=True)
    kc, kg = upload_cache(k, T, nf, nl)
    vc, vg = upload_cache(v, T, nf, nl)
    cap = kc["codes"].shape[2]
    ws = torch.full((gpu.attention_split_workspace_bytes(1, Hq, Nq, cap, split),), 0xFF,
                    dtype=torch.uint8, device="cuda:0")   # NaN patterns: every read slot is written
    ref, mag, bound, terms = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split, terms=True)
    for dt in (torch.float32, torch.bfloat16):
        O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg, out_dtype=dt, split=split,
                                   workspace=ws)
        torch.cuda.synchronize()
        got = to_host(O.float()).astype(np.float64)
        tol = T_.attention_tol(ref, mag, bound, terms, out_bf16=dt == torch.bfloat16)
        within(got, ref, tol, f"split kv cache {dt}")


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
    O = gpu.attention_kv_cache(upload(q), kc, kg, vc, vg, split=split)
    torch.cuda.synchronize()
    got = to_host(O).astype(np.float64)
    ref, mag, bound, terms = orc.attention_kv_cache(q, k, v, T, nf, nl, split=split, terms=True)
    within(got, ref, T_.attention_tol(ref, mag, bound, terms), "full-size decode")


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
