"""Independent NumPy brute force of NVFP4 ScaleSearch, used only to check the oracle.

Written separately from the C oracle (no shared code or tables): codecs are
nearest-value searches over value lists built from the bit layouts, and every
block is scored against all 127 finite E4M3 scale patterns, each SSE summed
with an explicit left-to-right loop over the 16 elements in float32.

Formats (pages: "NVIDIAのFP4推論が50倍の効率を実現" 超低精度推論を支えるアーキテクチャ;
BEVFormer B200 FP8/FP4 tuning article, 1-A and sec. 7): E2M1 = 1 sign, 2
exponent (bias 1), 1 mantissa bit; UE4M3 = 4 exponent (bias 7), 3 mantissa
bits, largest 448. Search: ScaleSearch summary page, 手法 > ScaleSearch.
"""
from __future__ import annotations

import numpy as np


def e2m1_values() -> np.ndarray:
    """Magnitudes of E2M1 codes 0..7 from the bit layout (exponent bias 1)."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals, dtype=np.float64)


def e4m3_values() -> np.ndarray:
    """Values of UE4M3 patterns 0..126 (127 is NaN) from the bit layout."""
    vals = []
    for p in range(127):
        e, m = p >> 3, p & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_G = e2m1_values()
_S = e4m3_values()


def e2m1_nearest(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code of y >= 0; exact halfway -> even code; y > 6 -> 7."""
    y = np.asarray(y, dtype=np.float32)
    yd = y.astype(np.float64)
    best = np.zeros(y.shape, dtype=np.int64)
    bestd = np.abs(yd - _G[0])
    for c in range(1, 8):
        d = np.abs(yd - _G[c])
        better = d < bestd
        tie = d == bestd
        take = better | (tie & (c % 2 == 0))
        best = np.where(take, c, best)
        bestd = np.where(take, d, bestd)
    # beyond the largest grid value the nearest is 6 (for huge y the float64
    # distances above can tie by rounding)
    best = np.where(yd >= _G[7], 7, best)
    return best


def e4m3_nearest(t: np.ndarray) -> np.ndarray:
    """Nearest UE4M3 pattern of t >= 0; exact halfway -> even pattern; t >= 448 -> 126."""
    t = np.asarray(t, dtype=np.float32).astype(np.float64)
    hi = np.searchsorted(_S, t, side="left")  # first value >= t
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = np.abs(t - _S[lo])
    dhi = np.abs(t - _S[hi])
    p = np.where(dlo < dhi, lo, hi)
    tie = (dlo == dhi) & (lo != hi)
    p = np.where(tie, np.where(lo % 2 == 0, lo, hi), p)
    p = np.where(t >= 448.0, 126, p)
    return p.astype(np.int64)


def sse_all_patterns(ax: np.ndarray, sg: np.float32) -> tuple[np.ndarray, np.ndarray]:
    """ax [nb, 16] float32 magnitudes -> (sse [nb, 127] float32, codes [nb, 127, 16])."""
    ax = np.asarray(ax, dtype=np.float32)
    nb = ax.shape[0]
    sse = np.empty((nb, 127), dtype=np.float32)
    codes = np.empty((nb, 127, 16), dtype=np.int8)
    sg = np.float32(sg)
    G32 = _G.astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore", under="ignore"):
        for p in range(127):
            d = np.float32(np.float32(_S[p]) * sg)
            r = np.float32(np.float32(1.0) / d)
            if np.isfinite(r):
                y = (ax * r).astype(np.float32)
                c = e2m1_nearest(y)
                xh = (G32[c] * d).astype(np.float32)
            else:
                c = np.zeros(ax.shape, dtype=np.int64)
                xh = np.zeros(ax.shape, dtype=np.float32)
            e = (ax - xh).astype(np.float32)
            q = (e * e).astype(np.float32)
            s = q[:, 0].copy()
            for i in range(1, 16):
                s = (s + q[:, i]).astype(np.float32)
            sse[:, p] = s
            codes[:, p, :] = c
    return sse, codes


def quantize_ref(x: np.ndarray, f_lo: int, f_hi: int, sg=None):
    """x [R, K] float32 (finite) -> (codes [R, K/2], scales [R, K/16], sg, chosen_f)."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    with np.errstate(over="ignore", under="ignore"):
        if sg is None:
            A = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
            sg = np.float32(A / np.float32(2688.0))
            if sg == 0:
                sg = np.float32(1.0)
        sg = np.float32(sg)
        blocks = x.reshape(-1, 16)
        ax = np.abs(blocks)
        amax = ax.max(axis=1)
        t = ((amax / np.float32(6.0)).astype(np.float32) / sg).astype(np.float32)
    p0 = e4m3_nearest(t)
    sse, allcodes = sse_all_patterns(ax, sg)
    nb = blocks.shape[0]
    order = [0] + [f for f in range(f_lo, f_hi + 1) if f != 0]
    best_p = p0.copy()
    best_s = sse[np.arange(nb), p0]
    best_f = np.zeros(nb, dtype=np.int64)
    for f in order[1:]:
        p = p0 + f
        ok = (p >= 0) & (p <= 126)
        pc = np.clip(p, 0, 126)
        s = sse[np.arange(nb), pc]
        win = ok & (s < best_s)
        best_p = np.where(win, pc, best_p)
        best_s = np.where(win, s, best_s)
        best_f = np.where(win, f, best_f)
    mag = allcodes[np.arange(nb), best_p, :].astype(np.uint8)
    sign = (np.signbit(blocks)).astype(np.uint8) << 3
    nib = (mag | sign).reshape(-1)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8).reshape(R, K // 2)
    scales = best_p.astype(np.uint8).reshape(R, K // 16)
    return codes, scales, sg, best_f.reshape(R, K // 16)


def sse_patterns(ax: np.ndarray, sg: np.float32, p: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """SSE of each block ax[b] under its own pattern p[b] (0..126) -> (sse [nb], codes [nb,16])."""
    ax = np.asarray(ax, dtype=np.float32)
    sg = np.float32(sg)
    G32 = _G.astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore", under="ignore"):
        d = (_S[p].astype(np.float32) * sg).astype(np.float32)
        r = (np.float32(1.0) / d).astype(np.float32)
        zero = ~np.isfinite(r)
        rr = np.where(zero, np.float32(0.0), r).astype(np.float32)
        y = (ax * rr[:, None]).astype(np.float32)
        c = e2m1_nearest(y)
        c = np.where(zero[:, None], 0, c)
        xh = (G32[c] * d[:, None]).astype(np.float32)
        xh = np.where(zero[:, None], np.float32(0.0), xh)
        e = (ax - xh).astype(np.float32)
        q = (e * e).astype(np.float32)
    s = q[:, 0].copy()
    for i in range(1, 16):
        s = (s + q[:, i]).astype(np.float32)
    return s, c


def quantize_ref_search(x: np.ndarray, f_lo: int, f_hi: int, sg=None):
    """Same result as quantize_ref, scoring only the candidates p0 + f (faster)."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    with np.errstate(over="ignore", under="ignore"):
        if sg is None:
            A = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
            sg = np.float32(A / np.float32(2688.0))
            if sg == 0:
                sg = np.float32(1.0)
        sg = np.float32(sg)
        blocks = x.reshape(-1, 16)
        ax = np.abs(blocks)
        amax = ax.max(axis=1)
        t = ((amax / np.float32(6.0)).astype(np.float32) / sg).astype(np.float32)
    p0 = e4m3_nearest(t)
    best_s, best_c = sse_patterns(ax, sg, p0)
    best_p = p0.copy()
    best_f = np.zeros(p0.shape, dtype=np.int64)
    for f in [f for f in range(f_lo, f_hi + 1) if f != 0]:
        p = p0 + f
        ok = (p >= 0) & (p <= 126)
        pc = np.clip(p, 0, 126)
        s, c = sse_patterns(ax, sg, pc)
        win = ok & (s < best_s)
        best_p = np.where(win, pc, best_p)
        best_s = np.where(win, s, best_s)
        best_f = np.where(win, f, best_f)
        best_c = np.where(win[:, None], c, best_c)
    sign = np.signbit(blocks).astype(np.uint8) << 3
    nib = (best_c.astype(np.uint8) | sign).reshape(-1)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8).reshape(R, K // 2)
    return codes, best_p.astype(np.uint8).reshape(R, K // 16), sg, best_f.reshape(R, K // 16)


# --- MXFP4 contrast format (32-element blocks, E8M0 power-of-two scales) ---

def mx_sse_all_exponents(ax: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """ax [nb, 32] float32 magnitudes -> (sse [nb, 255] float32 for X = -127..127,
    codes [nb, 255, 32])."""
    ax = np.asarray(ax, dtype=np.float32)
    nb = ax.shape[0]
    sse = np.empty((nb, 255), dtype=np.float32)
    codes = np.empty((nb, 255, 32), dtype=np.int8)
    G32 = _G.astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        for k, X in enumerate(range(-127, 128)):
            d = np.float32(2.0 ** X)
            r = np.float32(2.0 ** -X)
            y = (ax * r).astype(np.float32)
            c = e2m1_nearest(y)
            xh = (G32[c] * d).astype(np.float32)
            e = (ax - xh).astype(np.float32)
            q = (e * e).astype(np.float32)
            s = q[:, 0].copy()
            for i in range(1, 32):
                s = (s + q[:, i]).astype(np.float32)
            sse[:, k] = s
            codes[:, k, :] = c
    return sse, codes


def mx_quantize_ref(x: np.ndarray, f_lo: int, f_hi: int):
    """x [R, K] float32 (finite) -> (codes [R, K/2], scales [R, K/32] E8M0 bytes):
    every exponent scored, then the first strictly smaller SSE in the visiting
    order f = 0, f_lo..f_hi around X0 = floor(log2 amax) - 2."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    blocks = x.reshape(-1, 32)
    ax = np.abs(blocks)
    amax = ax.max(axis=1).astype(np.float64)
    with np.errstate(divide="ignore"):
        X0 = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    X0 = np.maximum(X0, -127).astype(np.int64)
    sse, allc = mx_sse_all_exponents(ax)
    nb = blocks.shape[0]
    rows = np.arange(nb)
    best_X = X0.copy()
    best_s = sse[rows, X0 + 127]
    for f in [f for f in range(f_lo, f_hi + 1) if f != 0]:
        X = X0 + f
        ok = (X >= -127) & (X <= 127)
        Xc = np.clip(X, -127, 127)
        s = sse[rows, Xc + 127]
        win = ok & (s < best_s)
        best_X = np.where(win, Xc, best_X)
        best_s = np.where(win, s, best_s)
    mag = allc[rows, best_X + 127, :].astype(np.uint8)
    sign = np.signbit(blocks).astype(np.uint8) << 3
    nib = (mag | sign).reshape(-1)
    codes = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8).reshape(R, K // 2)
    return codes, (best_X + 127).astype(np.uint8).reshape(R, K // 32)


# --- attention on NVFP4 operands ---

def nvfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [..., D/2], scales [..., D/16] -> float64 values V[code] * s (no tensor scale)."""
    c = np.asarray(codes, np.uint8)
    nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(*c.shape[:-1], c.shape[-1] * 2)
    mag = _G[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    s = _S[np.minimum(np.asarray(scales, np.int64), 126)]
    return mag * np.repeat(s, 16, axis=-1)


def attention_ref(q, k, v, tile: int = 32, causal: bool = False):
    """Same readings as the oracle's attention, written with NumPy: online softmax over
    key tiles, P coded per 16 keys by quantize_ref_search with S_P = fl(1/2688) and
    offsets [0, 0]. Returns O float64 [B, Hq, Nq, D]."""
    qd, kd, vd = (nvfp4_decode(t[0], t[1]) for t in (q, k, v))
    qg, kg, vg = (float(t[2]) for t in (q, k, v))
    B, Hq, Nq, D = qd.shape
    Hkv, Nk = kd.shape[1], kd.shape[2]
    SP = np.float32(1.0) / np.float32(2688.0)
    c = qg * kg / np.sqrt(D)
    O = np.zeros((B, Hq, Nq, D))
    for b in range(B):
        for h in range(Hq):
            Q = qd[b, h]
            K = kd[b, h // (Hq // Hkv)]
            V = vd[b, h // (Hq // Hkv)]
            S = (Q @ K.T) * c
            if causal:
                vis = np.arange(Nk)[None, :] <= (np.arange(Nq)[:, None] + Nk - Nq)
                S = np.where(vis, S, -np.inf)
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, D))
            for t0 in range(0, Nk, tile):
                St = np.full((Nq, tile), -np.inf)
                w = min(tile, Nk - t0)
                St[:, :w] = S[:, t0:t0 + w]
                mn = np.maximum(m, St.max(axis=1))
                live = mn > -np.inf
                with np.errstate(invalid="ignore"):
                    alpha = np.where(np.isfinite(m), np.exp(m - mn), 0.0)
                    P = np.where(np.isfinite(St), np.exp(St - mn[:, None]), 0.0).astype(np.float32)
                alpha = np.where(live, alpha, 1.0)
                P = np.where(live[:, None], P, np.float32(0))
                l = alpha * l + P.astype(np.float64).sum(axis=1)
                codes, scales, _, _ = quantize_ref_search(P, 0, 0, sg=SP)
                Ph = nvfp4_decode(codes, scales)
                Vt = np.zeros((tile, D))
                Vt[:w] = V[t0:t0 + w]
                acc = alpha[:, None] * acc + Ph @ Vt
                m = np.where(live, mn, m)
            with np.errstate(invalid="ignore", divide="ignore"):
                O[b, h] = np.where(l[:, None] > 0, acc * (float(SP) * vg) / l[:, None], 0.0)
    return O


def cache_values(c, T: int, nf: int, nl: int) -> np.ndarray:
    """[B, H, T, D] float64 values of the tokens a sink cache holds."""
    B, H = c["codes"].shape[:2]
    D = c["codes"].shape[3] * 2
    mid_hi = max(T - nl, nf)
    out = np.zeros((B, H, T, D))
    for t in range(T):
        if t < nf:
            w = np.asarray(c["head"][:, :, t], np.uint16)
        elif t >= mid_hi:
            w = np.asarray(c["tail"][:, :, t % nl], np.uint16)
        else:
            out[:, :, t] = nvfp4_decode(c["codes"][:, :, t - nf], c["scales"][:, :, t - nf]) * \
                float(c["gscale"])
            continue
        out[:, :, t] = (w.astype(np.uint32) << 16).view(np.float32)
    return out


def attention_cache_ref(q, k, v, T: int, nf: int, nl: int, tile: int = 32, split: int = 0):
    """Attention over the sink KV cache with NumPy: key values assembled from the head
    (t < nf), the ring (t >= max(nf, T - nl), slot t mod nl) and the coded middle; keys
    visited segment by segment in tiles of `tile` that stay inside a segment; P coded
    per 16 keys as in attention_ref. split > 0: the head, the tail and each piece of
    `split` middle tokens keep separate softmax states, merged at the end by the
    weights exp(m_u - max m)."""
    def bf(a):
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qd = nvfp4_decode(q[0], q[1]) * float(q[2])
    B, Hq, Nq, D = qd.shape
    Hkv = k["codes"].shape[1]
    mid_hi = max(T - nl, nf)
    SP = np.float32(1.0) / np.float32(2688.0)

    def values(c, b, hk):
        out = np.zeros((T, D))
        for t in range(T):
            if t < nf:
                out[t] = bf(c["head"][b, hk, t])
            elif t >= mid_hi:
                out[t] = bf(c["tail"][b, hk, t % nl])
            else:
                dec = nvfp4_decode(c["codes"][b, hk, t - nf], c["scales"][b, hk, t - nf])
                out[t] = dec * float(c["gscale"])
        return out

    segs = [(0, min(nf, T)), (nf, mid_hi), (max(mid_hi, nf), T)]
    if split:
        units = [[segs[0]], [segs[2]]] + [[(a, min(a + split, mid_hi))]
                                          for a in range(nf, mid_hi, split)]
    else:
        units = [segs]
    O = np.zeros((B, Hq, Nq, D))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            K, V = values(k, b, hk), values(v, b, hk)
            S = (qd[b, h] @ K.T) / np.sqrt(D)
            states = []
            for unit in units:
                m = np.full(Nq, -np.inf)
                l = np.zeros(Nq)
                acc = np.zeros((Nq, D))
                for lo, hi in unit:
                    for t0 in range(lo, hi, tile):
                        w = min(tile, hi - t0)
                        St = np.full((Nq, tile), -np.inf)
                        St[:, :w] = S[:, t0:t0 + w]
                        mn = np.maximum(m, St.max(axis=1))
                        with np.errstate(invalid="ignore"):
                            alpha = np.where(np.isfinite(m), np.exp(m - mn), 0.0)
                            P = np.where(np.isfinite(St), np.exp(St - mn[:, None]), 0.0).astype(np.float32)
                        l = alpha * l + P.astype(np.float64).sum(axis=1)
                        codes, scales, _, _ = quantize_ref_search(P, 0, 0, sg=SP)
                        Vt = np.zeros((tile, D))
                        Vt[:w] = V[t0:t0 + w]
                        acc = alpha[:, None] * acc + nvfp4_decode(codes, scales) @ Vt
                        m = mn
                states.append((m, l, acc))
            M = np.max([st[0] for st in states], axis=0)
            num = np.zeros((Nq, D))
            den = np.zeros(Nq)
            for m, l, acc in states:
                with np.errstate(invalid="ignore"):
                    wgt = np.where(np.isfinite(m), np.exp(m - M), 0.0)
                num += wgt[:, None] * acc
                den += wgt * l
            O[b, h] = num * float(SP) / den[:, None]
    return O
