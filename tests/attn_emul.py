"""A binary32 emulation of attention on NVFP4 operands, written apart from the oracle
(NumPy, its own order of operations), used on the CPU to check the bar the GPU
attention tests compare against (tests/attn_tol.py) from both sides:

- the emulation as it is (float32 scores from a float32 matrix product, float32
  exp, P coded per 16 keys by the NumPy quantizer reference, float32 products and
  sums in a two-pass order: each tile's sum of P^ v, then the tiles weighted by
  exp(m_tile - m_final)) stays inside the bar, and so do runs whose scores are
  moved by up to half the worst-case FP32 error of a 128-term dot product;
- runs with a planted structural mistake leave it: one key dropped, one 16-key
  block of P^ v dropped, tiles of 64 keys instead of 32, one P code one step off.

Readings are the oracle's (ScaleSearch summary page, ScaleSearchAttention):
online softmax over tiles, p = exp(s - m) against the running max, P coded per
16 keys with max scaling under S_P = fl(1/2688), O = S_P sum P^ v / l; sink keys
and values in bf16, coded ones as V[code] * s times their tensor scale.
"""
import numpy as np

import ref_numpy as R

F32 = np.float32
SP = F32(1) / F32(2688)
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MUTATIONS = ("drop_key", "drop_block", "tile64", "flip")


def _bf16(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def layout(units, tile):
    """Tiles of `tile` keys that stay inside each (lo, hi) range: key index per slot
    (-1 = padding) [n_tiles, tile], and the unit of each tile."""
    idx, unit_of = [], []
    for u, segs in enumerate(units):
        for lo, hi in segs:
            for t0 in range(lo, hi, tile):
                row = np.arange(t0, t0 + tile)
                idx.append(np.where(row < hi, row, -1))
                unit_of.append(u)
    if not idx:
        return np.zeros((0, tile), np.int64), np.zeros(0, np.int64)
    return np.array(idx), np.array(unit_of)


def run(S, V, units, tile=32, mutate=None, noise=None, rng=None):
    """O [R, D] (float32) of rows with scores S [R, N] (float32, natural-log units,
    -inf for keys a row does not see) over values V [N, D] (float32); `units` lists the
    key ranges of each softmax state (merged at the end). mutate: one of MUTATIONS,
    applied at the key of largest score of each row. noise: [R, N] largest score
    shift; each score moves by a uniform draw in [-noise/2, noise/2]. Returns O and
    P^ by key [R, N] (0 for keys a row does not see)."""
    S = np.array(S, dtype=F32, copy=True)
    Rn, N = S.shape
    rows = np.arange(Rn)
    tgt = np.argmax(S, axis=1) if N else np.zeros(Rn, np.int64)
    if noise is not None:
        S = (S + (rng.uniform(-0.5, 0.5, S.shape) * noise).astype(F32)).astype(F32)
    if mutate == "drop_key":
        S[rows, tgt] = -np.inf
    if mutate == "tile64":
        tile = 64
    idx, unit_of = layout(units, tile)
    nt = idx.shape[0]
    D = V.shape[1]
    if nt == 0:
        return np.zeros((Rn, D), F32), np.zeros((Rn, N), F32)
    valid = idx >= 0
    St = np.where(valid[None], S[:, np.maximum(idx, 0)], F32(-np.inf)).astype(F32)
    mt = St.max(axis=2)
    m = np.empty_like(mt)
    for u in np.unique(unit_of):
        sl = np.flatnonzero(unit_of == u)
        m[:, sl] = np.maximum.accumulate(mt[:, sl], axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        arg = (St - m[..., None]).astype(F32)
        p = np.where(np.isfinite(St) & np.isfinite(m[..., None]), np.exp(arg), F32(0)).astype(F32)
    codes, scales, _, _ = R.quantize_ref_search(p.reshape(-1, tile), 0, 0, sg=SP)
    Ph = R.nvfp4_decode(codes, scales).astype(F32).reshape(Rn, nt, tile)
    if mutate in ("drop_block", "flip"):
        for r in range(Rn):
            t, e = np.argwhere(idx == tgt[r])[0]
            if mutate == "drop_block":
                Ph[r, t, (e // 16) * 16:(e // 16) * 16 + 16] = 0
            else:
                s = R.e4m3_values()[scales.reshape(Rn, nt, tile // 16)[r, t, e // 16]]
                c = int(np.argmin(np.abs(GRID * s - Ph[r, t, e])))
                Ph[r, t, e] = F32(GRID[6 if c == 7 else c + 1] * s)
    Pk = np.zeros((Rn, N), F32)                          # P^ by key (0 where unseen)
    flat = idx.reshape(-1)
    Pk[:, flat[flat >= 0]] = Ph.reshape(Rn, -1)[:, flat >= 0]
    Vt = np.where(valid[..., None], V[np.maximum(idx, 0)], F32(0)).astype(F32)
    C = np.matmul(Ph.transpose(1, 0, 2), Vt)            # [nt, R, D]: each tile's sum of P^ v
    ps = p.sum(axis=2, dtype=F32)                        # [R, nt]
    num = np.zeros((Rn, D), F32)
    den = np.zeros(Rn, F32)
    Mu, accs, ls = [], [], []
    for u in np.unique(unit_of):
        sl = np.flatnonzero(unit_of == u)
        M = m[:, sl[-1]]
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(m[:, sl]), np.exp((m[:, sl] - M[:, None]).astype(F32)),
                         F32(0)).astype(F32)
        accs.append(np.einsum("rt,trd->rd", w, C[sl]).astype(F32))
        ls.append((w * ps[:, sl]).sum(axis=1, dtype=F32))
        Mu.append(M)
    Mu = np.stack(Mu)
    Mall = Mu.max(axis=0)
    for M, acc, l in zip(Mu, accs, ls):
        with np.errstate(invalid="ignore"):
            W = np.where(np.isfinite(M), np.exp((M - Mall).astype(F32)), F32(0)).astype(F32)
        num = (num + W[:, None] * acc).astype(F32)
        den = (den + W * l).astype(F32)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(den[:, None] > 0, (num * SP) / den[:, None], F32(0)).astype(F32)
    return O, Pk


def dot_error(Qd, K, cf):
    """Worst-case FP32 error of each score: 128 u sum |q_d k_d| times the key's score
    factor (the textbook bound of a 128-term dot product in binary32)."""
    return (128 * 2.0 ** -24 * (np.abs(Qd).astype(np.float64) @ np.abs(K).astype(np.float64).T) *
            np.abs(cf)[None, :]).astype(F32)


def prefill_inputs(q, k, v, b, hk, Hq, Hkv, causal=False, rows=None):
    """Scores, values and units of the query rows of KV head hk of batch b (all query
    heads that share it), for the plain attention."""
    qd = R.nvfp4_decode(q[0], q[1]).astype(F32)
    Kd = R.nvfp4_decode(k[0][b, hk], k[1][b, hk]).astype(F32)
    Vd = (R.nvfp4_decode(v[0][b, hk], v[1][b, hk]).astype(F32) * F32(v[2])).astype(F32)
    G = Hq // Hkv
    Qg = qd[b, hk * G:(hk + 1) * G]                      # [G, Nq, D]
    Nq, Nk = Qg.shape[1], Kd.shape[0]
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    Qr = Qg[:, sel].reshape(-1, Qg.shape[-1])
    cf = np.full(Nk, F32(F32(q[2]) * F32(k[2])) * F32(1.0 / np.sqrt(128.0)), F32)
    S = (np.matmul(Qr, Kd.T) * cf[None, :]).astype(F32)
    if causal:
        i = np.tile(sel, G)
        S = np.where(np.arange(Nk)[None, :] <= (i[:, None] + Nk - Nq), S, F32(-np.inf))
    return S, Vd, [[(0, Nk)]], dot_error(Qr, Kd, cf)


def cache_inputs(q, kc, vc, T, nf, nl, hk, Hq, Hkv, split=0):
    """The same for the sink cache of KV head hk (batch 0): head keys, the coded middle
    and the tail ring, in token order; units as the split reading lays them out."""
    qd = R.nvfp4_decode(q[0], q[1]).astype(F32)
    D = qd.shape[-1]
    mid_hi = max(T - nl, nf)
    K = np.zeros((T, D), F32)
    Vv = np.zeros((T, D), F32)
    cf = np.zeros(T, F32)
    tau = F32(1.0 / np.sqrt(128.0))
    head = np.arange(min(nf, T))
    tail = np.arange(max(mid_hi, nf), T)
    mid = np.arange(nf, mid_hi)
    for idx, src in ((head, lambda c: c["head"][0, hk, head]),
                     (tail, lambda c: c["tail"][0, hk, tail % max(nl, 1)])):
        if idx.size:
            K[idx], Vv[idx] = _bf16(src(kc)), _bf16(src(vc))
            cf[idx] = F32(F32(q[2]) * tau)
    if mid.size:
        K[mid] = R.nvfp4_decode(kc["codes"][0, hk, mid - nf], kc["scales"][0, hk, mid - nf])
        Vv[mid] = (R.nvfp4_decode(vc["codes"][0, hk, mid - nf], vc["scales"][0, hk, mid - nf]) *
                   float(vc["gscale"])).astype(F32)
        cf[mid] = F32(F32(F32(q[2]) * F32(kc["gscale"])) * tau)
    G = Hq // Hkv
    Qr = qd[0, hk * G:(hk + 1) * G].reshape(-1, D)
    S = (np.matmul(Qr, K.T) * cf[None, :]).astype(F32)
    segs = [(0, min(nf, T)), (nf, mid_hi), (max(mid_hi, nf), T)]
    if split:
        units = [[segs[0]], [segs[2]]] + [[(a, min(a + split, mid_hi))]
                                          for a in range(nf, mid_hi, split)]
    else:
        units = [segs]
    return S, Vv, units, dot_error(Qr, K, cf)
