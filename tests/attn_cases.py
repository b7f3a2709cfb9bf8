"""Seeded operands of the attention tests (the GPU parity tests and the CPU tests of
their comparison bound build the same cases). Every operand is coded by the oracle;
nothing here comes from the HIP path."""
import numpy as np

import workloads


def coded(orc, x):
    """(codes [..., 64], scales [..., 8], tensor scale) of a [..., 128] tensor, ScaleSearch
    offsets [-2, 6]."""
    c, s, g = orc.quantize(x, -2, 6)
    shp = x.shape[:-1]
    return c.reshape(*shp, 64), s.reshape(*shp, 8), g


def make_ops(orc, B, Hq, Hkv, Nq, Nk, seed):
    """Q N(0, 1), K of the KV-cache workload recipe, V N(0, 1), all bf16, coded."""
    rng = np.random.default_rng(seed)
    q = workloads.to_bf16_bits(rng.standard_normal((B, Hq, Nq, 128)).astype(np.float32))
    k = workloads.workload(3, (B, Hkv, Nk, 128))
    v = workloads.to_bf16_bits(rng.standard_normal((B, Hkv, Nk, 128)).astype(np.float32))
    return coded(orc, q), coded(orc, k), coded(orc, v)


def hadamard_ops(orc):
    """Q and K coded after the same randomized Hadamard transform (offsets [-8, 8])."""
    rng = np.random.default_rng(8)
    signs = rng.integers(0, 2**32, 4, dtype=np.uint64).astype(np.uint32)
    qx = workloads.workload(5, (1, 4, 200, 128))
    kx = workloads.workload(3, (1, 1, 700, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, 1, 700, 128)).astype(np.float32))

    def rht(x):
        c, s, g = orc.quantize_rht(x, signs, -8, 8)
        return c.reshape(*x.shape[:-1], 64), s.reshape(*x.shape[:-1], 8), g

    return rht(qx), rht(kx), coded(orc, vx)


def full_size_ops(orc, rows=None):
    """The 32K benchmark operands: Q [1, 32, 32768, 128] (Q workload recipe), K
    [1, 8, 32768, 128] (KV workload recipe), V N(0, 1). rows (optional): code only these query rows
    of Q, under the whole tensor's scale (blocks are coded independently, so these are
    the same bytes as those rows of the whole tensor's coding)."""
    rng = np.random.default_rng(17)
    qx = workloads.workload(5)
    kx = workloads.workload(3)
    vx = workloads.to_bf16_bits(rng.standard_normal(kx.shape).astype(np.float32))
    if rows is None:
        q = coded(orc, qx)
    else:
        g = np.float32(np.float32(np.abs(workloads.bf16_bits_to_f32(qx)).max()) / np.float32(2688))
        sub = np.ascontiguousarray(qx[:, :, rows])
        c, s, _ = orc.quantize(sub, -2, 6, gscale=float(g))
        q = (c.reshape(*sub.shape[:-1], 64), s.reshape(*sub.shape[:-1], 8), g)
    return q, coded(orc, kx), coded(orc, vx)


def sampled_rows():
    """Query rows the full-size test compares: four drawn from a seeded generator, plus
    the first and the last."""
    rows = np.sort(np.random.default_rng(18).choice(32768, 4, replace=False))
    return np.unique(np.concatenate([rows, [0, 32767]]))


def cache_of(orc, x, nf, nl, T, cap):
    """Sink-cache buffers of a [B, H, T, D] bf16 tensor, as the KV append builds them."""
    B, H, _, D = x.shape
    mid = max(T - nf - nl, 0)
    g = np.float32(np.abs(workloads.bf16_bits_to_f32(x[:, :, nf:T - nl])).max() / 2688) if mid else np.float32(1)
    c, s, _ = orc.quantize(np.ascontiguousarray(x[:, :, nf:nf + mid]).reshape(-1, D) if mid else
                           np.zeros((0, D), np.uint16), -2, 6, gscale=float(g))
    codes = np.zeros((B, H, cap, D // 2), np.uint8)
    scales = np.zeros((B, H, cap, D // 16), np.uint8)
    codes[:, :, :mid] = c.reshape(B, H, mid, D // 2)
    scales[:, :, :mid] = s.reshape(B, H, mid, D // 16)
    head = np.zeros((B, H, nf, D), np.uint16)
    head[:, :, :min(nf, T)] = x[:, :, :min(nf, T)]
    tail = np.zeros((B, H, nl, D), np.uint16)
    for t in range(max(nf, T - nl), T):
        tail[:, :, t % nl] = x[:, :, t]
    return dict(head=head, tail=tail, codes=codes, scales=scales, gscale=g)


def cache_case(orc, Hq, Hkv, Nq, T, nf, nl, seed):
    """Q coded by the oracle and K, V sink caches built by the oracle (cap = middle + 8)."""
    rng = np.random.default_rng(seed)
    qx = workloads.to_bf16_bits(rng.standard_normal((1, Hq, Nq, 128)).astype(np.float32))
    kx = workloads.workload(3, (1, Hkv, T, 128))
    vx = workloads.to_bf16_bits(rng.standard_normal((1, Hkv, T, 128)).astype(np.float32))
    q = coded(orc, qx)
    cap = max(T - nf - nl, 0) + 8
    return q, cache_of(orc, kx, nf, nl, T, cap), cache_of(orc, vx, nf, nl, T, cap)


# the shapes the GPU parity tests run (B, Hq, Hkv, Nq, Nk)
PREFILL_SHAPES = [(1, 2, 1, 300, 1000), (2, 1, 1, 128, 32), (1, 4, 2, 77, 513), (1, 1, 1, 1, 5)]
CAUSAL_SHAPES = [(257, 257), (100, 300), (300, 100)]   # (Nq, Nk), one batch, 2 heads
CACHE_SHAPES = [(2, 1, 77, 1000, 128, 128), (4, 2, 40, 300, 64, 0), (1, 1, 33, 90, 64, 64),
                (1, 1, 20, 50, 64, 16), (2, 2, 64, 200, 0, 0), (1, 1, 5, 520, 32, 96),
                (8, 1, 17, 300, 16, 16)]               # (Hq, Hkv, Nq, T, nf, nl)
SPLIT_SHAPES = [(32, 8, 1, 3000, 128, 128, 256), (4, 2, 40, 300, 64, 0, 64),
                (1, 1, 5, 520, 32, 96, 96), (2, 1, 3, 50, 64, 16, 32), (2, 2, 1, 200, 0, 0, 32),
                (8, 1, 16, 700, 16, 16, 128), (8, 1, 17, 700, 16, 16, 128)]
