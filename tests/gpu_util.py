"""Helpers for the GPU parity tests: host <-> device transfers of the seeded inputs."""
import numpy as np
import torch


def to_dev(x: np.ndarray, dev="cuda:0") -> torch.Tensor:
    """float32 -> torch.float32; uint16 (bf16 bits) -> torch.bfloat16."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    if x.dtype == np.float32:
        return torch.from_numpy(x).to(dev)
    raise TypeError(x.dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_same_floats(got: np.ndarray, ref: np.ndarray):
    """Bit-exact equality, except that any NaN matches any NaN (payloads unspecified)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.dtype == np.uint16:
        gn = (got & 0x7FFF) > 0x7F80
        rn = (ref & 0x7FFF) > 0x7F80
        gb, rb = got, ref
    else:
        gn, rn = np.isnan(got), np.isnan(ref)
        gb, rb = f32_bits(got), f32_bits(ref)
    np.testing.assert_array_equal(gn, rn)
    bad = (gb != rb) & ~rn
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:8]
        raise AssertionError(f"{bad.sum()} mismatches; first at {i}: got "
                             f"{gb.reshape(-1)[i]} want {rb.reshape(-1)[i]}")


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    d = np.flatnonzero((np.asarray(a) != np.asarray(b)).reshape(-1))
    if d.size == 0:
        return "none"
    return f"{d.size} differ; first flat index {d[0]}: {a.reshape(-1)[d[0]]} vs {b.reshape(-1)[d[0]]}"
