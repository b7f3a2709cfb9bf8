"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds only input generation: NumPy PCG64 draws, the outlier
recipes, and the cast of the draws to the stored dtype. It holds none of the
quantizer's arithmetic and imports neither the oracle nor the product.

bf16 tensors are returned as ``uint16`` arrays of bfloat16 bit patterns
(round-to-nearest-even of the float32 value); FP32 tensors as ``float32``.

The five workloads stand in for what the ScaleSearch summary page measures on
(Llama 3.1 Key states, LLM and diffusion weights/activations, 32K-token
attention Q/K), which are model weights and datasets this project does not
have. Shapes and distributions:

1. FP32 1024 x 1024, i.i.d. N(0, 1).
2. bf16 4096 x 4096, 0.5 * Student-t(3), 1% of columns (41 of 4096, drawn
   without replacement) multiplied by 50 as outlier channels.
3. bf16 KV-cache K [1, 8, 32768, 128]: N(0, 1) times a per-(head, channel)
   log-normal(0, 0.5) factor shared over tokens; sink mode 128 + 128 tokens.
4. bf16 weight 8192 x 28672, N(0, 0.02^2).
5. bf16 Q [1, 32, 32768, 128]: N(0, 1), i.i.d. Bernoulli(0.001) entries x 30;
   128-point Hadamard then offsets [-8, 8].

Seed = workload index - 1 (PCG64 ``default_rng``). Smaller variants keep the
recipe and change only the leading (row/token/head) sizes.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_bf16_bits", "bf16_bits_to_f32", "workload", "WORKLOADS", "device_gaussian_planted",
]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def gaussian_f32(shape, seed: int) -> np.ndarray:
    """Workload 1: N(0, 1) drawn in float64 and cast to float32."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape).astype(np.float32)


def student_t_outlier_cols(shape, seed: int) -> np.ndarray:
    """Workload 2: 0.5 * t(3), round(1% of columns) x 50, bf16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, shape)
    x *= 0.5
    ncols = shape[-1]
    k = int(round(0.01 * ncols))
    cols = rng.choice(ncols, size=k, replace=False)
    x[..., cols] *= 50.0
    return to_bf16_bits(x.astype(np.float32))


def kv_lognormal_channels(shape, seed: int) -> np.ndarray:
    """Workload 3: N(0, 1) * lognormal(0, 0.5) per (head, channel), bf16 bits."""
    B, H, T, D = shape
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    scale = rng.lognormal(0.0, 0.5, (1, H, 1, D))
    x *= scale
    return to_bf16_bits(x.astype(np.float32))


def weight_gaussian(shape, seed: int) -> np.ndarray:
    """Workload 4: N(0, 0.02^2), bf16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    x *= 0.02
    return to_bf16_bits(x.astype(np.float32))


def q_sparse_outliers(shape, seed: int) -> np.ndarray:
    """Workload 5: N(0, 1) with i.i.d. Bernoulli(0.001) entries x 30, bf16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    mask = rng.random(shape) < 0.001
    x[mask] *= 30.0
    return to_bf16_bits(x.astype(np.float32))


def device_gaussian_planted(rows: int, cols: int, seed: int, dtype, device, peak: float = 8.0,
                            row: int | None = None):
    """A tensor too large to draw on the host: N(0, 1) drawn on the device by torch's
    seeded generator directly in ``dtype`` (torch.bfloat16 or torch.float32), clamped
    to [-peak/2, peak/2], with element [row, 5] (default: the last row) set to
    ``peak``, so that the tensor's largest magnitude is ``peak`` by construction.
    Returns the device tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, dtype=dtype, device=device)
    x.clamp_(-peak / 2, peak / 2)
    x[rows - 1 if row is None else row, 5] = peak
    return x


# name -> (generator, full shape, seed, description of the mode)
WORKLOADS = {
    1: dict(gen=gaussian_f32, shape=(1024, 1024), seed=0, dtype="f32", offsets=(-2, 6),
            hadamard=False, sink=None,
            name="fp32 1024x1024 N(0,1), blocks of 16, offsets [-2,6]"),
    2: dict(gen=student_t_outlier_cols, shape=(4096, 4096), seed=1, dtype="bf16",
            offsets=(-2, 6), hadamard=False, sink=None,
            name="bf16 4096x4096 0.5*t(3) with 41 outlier columns x50, offsets [-2,6]"),
    3: dict(gen=kv_lognormal_channels, shape=(1, 8, 32768, 128), seed=2, dtype="bf16",
            offsets=(-2, 6), hadamard=False, sink=(128, 128),
            name="bf16 KV K [1,8,32768,128] N(0,1)*lognormal(0,0.5) channels, sink 128+128"),
    4: dict(gen=weight_gaussian, shape=(8192, 28672), seed=3, dtype="bf16", offsets=(-2, 6),
            hadamard=False, sink=None,
            name="bf16 weight 8192x28672 N(0,0.02^2), offsets [-2,6]"),
    5: dict(gen=q_sparse_outliers, shape=(1, 32, 32768, 128), seed=4, dtype="bf16",
            offsets=(-8, 8), hadamard=True, sink=None,
            name="bf16 Q [1,32,32768,128] N(0,1) 0.1% x30, Hadamard-128, offsets [-8,8]"),
}


def workload(idx: int, shape=None) -> np.ndarray:
    """Generate workload ``idx`` at its full shape or at ``shape`` (same recipe)."""
    w = WORKLOADS[idx]
    return w["gen"](tuple(shape) if shape is not None else w["shape"], w["seed"])
