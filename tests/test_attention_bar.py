"""The bar the GPU attention tests compare against (tests/attn_tol.py, computed from
the oracle's terms), checked on the CPU from both sides at every shape those tests
run, the full 32K shapes included (ScaleSearch summary page, ScaleSearchAttention,
ネイティブ NVFP4 実行: QK^T and PV on NVFP4 operands with FP32 accumulation).

Against a binary32 emulation written apart from the oracle (tests/attn_emul.py):
- not too tight: the emulation stays inside the bar, and so do runs whose scores
  are moved by up to half the worst-case FP32 error of a 128-term dot product
  (P codes near a rounding midpoint then flip: the runs check that some do, and
  that the oracle's flip allowance covers them);
- not too loose: the emulation with one planted mistake leaves the bar: the key of
  largest score dropped, the 16-key block of P^ v holding it dropped, that key's P
  code one step off (away from any midpoint: it codes its block's max), and tiles
  of 64 keys instead of 32 (wherever the 64-key tiling computes something else).
"""
import numpy as np
import pytest

import attn_cases as AC
import attn_emul as E
import attn_tol as T


SEEDS = (1, 2, 3)   # perturbed runs per row group


def check(groups, flips_expected=True):
    """groups: (S, V, units, de, oracle rows, bar rows) per KV head. Every run's worst
    |emulated - oracle| / bar, then the assertions of the module docstring."""
    worst = {}
    recoded = False  # does the 64-key tiling code any P differently?
    flips = 0
    for (S, V, units, de, ref, tol) in groups:
        clean, P0 = E.run(S, V, units)
        outs = {"clean": clean}
        for sd in SEEDS:
            pert, P1 = E.run(S, V, units, noise=de, rng=np.random.default_rng(sd))
            outs[f"perturbed{sd}"] = pert
            flips += int(np.sum(P0 != P1))
        for m in E.MUTATIONS:
            outs[m], Pm = E.run(S, V, units, mutate=m)
            if m == "tile64":
                recoded |= not np.array_equal(Pm, P0)
        for name, got in outs.items():
            r = float(np.max(np.abs(got.astype(np.float64) - ref) / np.maximum(tol, 1e-300),
                             initial=0.0))
            worst[name] = max(worst.get(name, 0.0), r)
    print({k: round(v, 4) for k, v in worst.items()}, f"P codes flipped by the perturbation: {flips}")
    assert worst["clean"] <= 1.0
    for sd in SEEDS:
        assert worst[f"perturbed{sd}"] <= 1.0
    for m in E.MUTATIONS:
        if m == "tile64" and not recoded:
            continue  # no P coded differently: the same computation up to sum order
        assert worst[m] > 1.0, f"mutation {m} stays inside the bar ({worst[m]:.3f})"
    if flips_expected:
        assert flips > 0, "the perturbed scores flipped no P code: they test nothing"
    return worst


def prefill_groups(orc, q, k, v, causal=False, out_bf16=False):
    O, mag, bound, terms = orc.attention_nvfp4(q, k, v, causal=causal, terms=True)
    tol = T.attention_tol(O, mag, bound, terms, out_bf16=out_bf16)
    B, Hq = q[0].shape[:2]
    Hkv = k[0].shape[1]
    G, D = Hq // Hkv, O.shape[-1]
    groups = []
    for b in range(B):
        for hk in range(Hkv):
            S, V, units, de = E.prefill_inputs(q, k, v, b, hk, Hq, Hkv, causal)
            hs = slice(hk * G, (hk + 1) * G)
            groups.append((S, V, units, de, O[b, hs].reshape(-1, D), tol[b, hs].reshape(-1, D)))
    return groups


def cache_groups(orc, q, kc, vc, T_, nf, nl, split=0):
    O, mag, bound, terms = orc.attention_kv_cache(q, kc, vc, T_, nf, nl, split=split, terms=True)
    tol = T.attention_tol(O, mag, bound, terms)
    Hq = q[0].shape[1]
    Hkv = kc["codes"].shape[1]
    G, D = Hq // Hkv, O.shape[-1]
    groups = []
    for hk in range(Hkv):
        S, V, units, de = E.cache_inputs(q, kc, vc, T_, nf, nl, hk, Hq, Hkv, split)
        hs = slice(hk * G, (hk + 1) * G)
        groups.append((S, V, units, de, O[0, hs].reshape(-1, D), tol[0, hs].reshape(-1, D)))
    return groups


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk", AC.PREFILL_SHAPES)
def test_prefill_bar(orc, B, Hq, Hkv, Nq, Nk):
    q, k, v = AC.make_ops(orc, B, Hq, Hkv, Nq, Nk, seed=Nq + Nk)
    check(prefill_groups(orc, q, k, v), flips_expected=B * Hq * Nq * Nk >= 40000)


@pytest.mark.parametrize("Nq,Nk", AC.CAUSAL_SHAPES)
def test_causal_bar(orc, Nq, Nk):
    q, k, v = AC.make_ops(orc, 1, 2, 2, Nq, Nk, seed=Nq * 3 + Nk)
    check(prefill_groups(orc, q, k, v, causal=True), flips_expected=Nq * Nk >= 40000)


def test_bf16_output_bar(orc):
    q, k, v = AC.make_ops(orc, 1, 1, 1, 200, 400, seed=3)
    check(prefill_groups(orc, q, k, v, out_bf16=True))


def test_hadamard_operands_bar(orc):
    check(prefill_groups(orc, *AC.hadamard_ops(orc)))


@pytest.mark.parametrize("Hq,Hkv,Nq,T_,nf,nl", AC.CACHE_SHAPES)
def test_cache_bar(orc, Hq, Hkv, Nq, T_, nf, nl):
    q, kc, vc = AC.cache_case(orc, Hq, Hkv, Nq, T_, nf, nl, T_ + 7 * nf + nl)
    check(cache_groups(orc, q, kc, vc, T_, nf, nl), flips_expected=Hq * Nq * T_ >= 40000)


@pytest.mark.parametrize("Hq,Hkv,Nq,T_,nf,nl,split", AC.SPLIT_SHAPES)
def test_split_cache_bar(orc, Hq, Hkv, Nq, T_, nf, nl, split):
    q, kc, vc = AC.cache_case(orc, Hq, Hkv, Nq, T_, nf, nl, T_ + split + Nq)
    check(cache_groups(orc, q, kc, vc, T_, nf, nl, split), flips_expected=Hq * Nq * T_ >= 40000)


def test_full_size_prefill_bar(orc):
    """The 32K benchmark shape (Q 32 heads, K/V 8 heads, non-causal) on the rows the GPU
    test samples: every mistake leaves the bar, the 64-key tiling by the smallest margin
    (1.6 of the bar): it recodes the P of ~1.5% of the keys (those before a rise of the
    running max), whose weight is small at 32K keys, while the bar here is dominated by
    the allowance for P codes that worst-case binary32 scores could round the other
    way. On the rows of another draw that mistake came to 0.71 of the bar, inside it."""
    rows = AC.sampled_rows()
    q, k, v = AC.full_size_ops(orc, rows=rows)
    check(prefill_groups(orc, q, k, v))


@pytest.mark.parametrize("split", [160, 512])
def test_full_size_decode_bar(orc, split):
    """One decode query per head (32 over 8 KV heads), a cache of 128 + 32768 + 128
    tokens split into pieces of 160 and 512: every mistake leaves the bar."""
    Hq, Hkv, Nq, nf, nl = 32, 8, 1, 128, 128
    T_ = nf + 32768 + nl
    q, kc, vc = AC.cache_case(orc, Hq, Hkv, Nq, T_, nf, nl, 2024)
    check(cache_groups(orc, q, kc, vc, T_, nf, nl, split))
