"""Python binding of libnvfp4.so (the C ABI in include/nvfp4.h).

Argument marshalling only: every step of the quantizer runs in the library's
HIP kernels. torch supplies device memory and the current HIP stream. There is
no CPU fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

F32, BF16 = 0, 1
HADAMARD128, GSCALE_GIVEN, PAIR_Q = 1, 2, 4

STATUS = {0: "NVFP4_OK", 1: "NVFP4_EINVAL", 2: "NVFP4_ESHAPE", 3: "NVFP4_EALIGN",
          4: "NVFP4_EWORKSPACE", 5: "NVFP4_EHIP"}

# exported symbol -> (argtypes, restype)
_i64, _i32, _u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "nvfp4_status_str": ([_i32], ctypes.c_char_p),
    "nvfp4_abi_version": ([], _i32),
    "nvfp4_hw_self_check": ([_vp], _i32),
    "nvfp4_workspace_bytes": ([_i64, _i64, _u32], _sz),
    "nvfp4_quantize": ([_vp, _i32, _i64, _i64, _i32, _i32, _i32, _u32, _vp, _vp, _vp, _vp, _sz,
                        _vp], _i32),
    "nvfp4_quantize_noalloc": ([_vp, _i32, _i64, _i64, _i32, _i32, _i32, _u32, _vp, _vp, _vp,
                                _vp], _i32),
    "nvfp4_noalloc_scratch_bytes": ([], _sz),
    "nvfp4_balance_workspace_bytes": ([_i64], _sz),
    "nvfp4_balance_exponents": ([_vp, _vp, _i32, _i64, _i64, _i64, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_quantize_balanced": ([_vp, _i32, _i64, _i64, _i32, _i32, _i32, _u32, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_hadamard128_balanced": ([_vp, _i32, _i64, _vp, _u32, _vp, _vp, _vp], _i32),
    "nvfp4_global_scale": ([_vp, _i32, _i64, _i64, _u32, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_dequantize": ([_vp, _vp, _vp, _i64, _i64, _i32, _vp, _i32, _vp], _i32),
    "nvfp4_quantize_kv_sink": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                _u32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_dequantize_kv_sink": ([_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _i32, _vp, _i32, _vp], _i32),
    "nvfp4_hadamard128": ([_vp, _i32, _i64, _vp, _vp], _i32),
    "nvfp4_kv_append": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _i32,
                         _i32, _u32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "nvfp4_kv_append_dev": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _i32,
                             _i32, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "nvfp4_kv_append2_dev": ([_vp, _vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32,
                              _i32, _i32, _vp], _i32),
    "nvfp4_quantize_rht": ([_vp, _i32, _i64, _i64, _i32, _i32, _i32, _u32, _vp, _vp, _vp, _vp,
                            _vp, _sz, _vp], _i32),
    "nvfp4_global_scale_rht": ([_vp, _i32, _i64, _i64, _u32, _vp, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_quantize_kv_sink_rht": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _i32,
                                    _i32, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "nvfp4_kv_append_rht": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32,
                             _i32, _i32, _u32, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "nvfp4_hadamard128_rht": ([_vp, _i32, _i64, _vp, _vp, _vp], _i32),
    "nvfp4_attention": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                         _i64, _i64, _i32, _vp, _i32, _vp], _i32),
    "nvfp4_attention_kv_cache": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _vp, _i32, _vp], _i32),
    "nvfp4_attention_kv_cache_dev": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _i32, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                      _i64, _vp, _i32, _vp], _i32),
    "nvfp4_attention_kv_cache_split": ([_vp] * 13 + [_i32, _i64, _i64, _i64, _i64, _i64, _i64,
                                        _i64, _i64, _i64, _i64, _vp, _sz, _vp, _i32, _vp], _i32),
    "nvfp4_attention_kv_cache_split_dev": ([_vp] * 13 + [_i32, _i64, _i64, _i64, _i64, _vp, _i64,
                                            _i64, _i64, _i64, _i64, _vp, _sz, _vp, _i32, _vp],
                                           _i32),
    "nvfp4_attention_split_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64], _sz),
    "mxfp4_quantize": ([_vp, _i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "mxfp4_dequantize": ([_vp, _vp, _i64, _i64, _i32, _vp, _i32, _vp], _i32),
}

_lock = threading.Lock()
_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


def load() -> ctypes.CDLL:
    """Load libnvfp4.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run microscaling_fp4_block_amd/build.py "
                    "(or __graft_entry__.build()) first")
            L = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _lib = L
    return _lib


def _check(fn: str, st: int):
    if st != 0:
        if st in (1, 2, 3, 4):
            raise ValueError(f"{fn}: {STATUS.get(st, st)}")
        raise NVFP4Error(fn, st)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors must be on a HIP (cuda) device")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.device


def _expect(t: torch.Tensor, name: str, shape, dtype, dev):
    """A caller-supplied tensor the kernels read or write: on the same device,
    contiguous, of this dtype and exactly this shape (so no access leaves it)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    return t


def _scale_arg(g: torch.Tensor, name: str, dev):
    """A device float32 tensor scale of one element."""
    _expect(g, name, None, torch.float32, dev)
    if g.numel() != 1:
        raise ValueError(f"{name} must hold one element")
    return g


def _workspace(ws, nbytes: int, dev):
    """The caller's workspace (any contiguous device tensor of at least nbytes bytes)
    or a new one; returns (tensor, its size in bytes)."""
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _expect(ws, "workspace", None, None, dev)
    return ws, ws.numel() * ws.element_size()


def workspace_bytes(rows: int, cols: int, flags: int = 0) -> int:
    return int(load().nvfp4_workspace_bytes(rows, cols, flags))


def hw_self_check() -> tuple:
    """nvfp4_hw_self_check on the current device: (values in [0, 448] whose hardware
    FP32 -> FP8 convert differs from the UE4M3 nearest-even rounding, scale bytes
    0..126 whose hardware FP8 -> FP32 convert differs from their UE4M3 value)."""
    counts = (ctypes.c_int64 * 2)()
    _check("nvfp4_hw_self_check", load().nvfp4_hw_self_check(ctypes.addressof(counts)))
    return int(counts[0]), int(counts[1])


def _signs(signs):
    """Random signs of the randomized Hadamard transform as a host uint32[4]
    (bit k % 32 of word k // 32 negates feature k); None for the plain transform."""
    if signs is None:
        return None
    if isinstance(signs, torch.Tensor):
        signs = signs.cpu().tolist()
    w = [int(v) for v in signs]
    if len(w) != 4 or any(v < 0 or v >= 1 << 32 for v in w):
        raise ValueError("signs: four uint32 words")
    return (ctypes.c_uint32 * 4)(*w)


def _offsets(offsets):
    lo, hi = int(offsets[0]), int(offsets[1])
    return lo, hi


def _balance(balance, K, dev):
    """(channel exponents, side) of the balancing pair: a device int8 tensor of K
    exponents (16-byte aligned, contiguous) and "q" or "k"; returns (pointer, flag)."""
    e, side = balance
    _expect(e, "balance exponents", (K,), torch.int8, dev)
    if e.data_ptr() % 16:
        raise ValueError("balance exponents must be 16-byte aligned")
    if side not in ("q", "k"):
        raise ValueError('balance side must be "q" or "k"')
    return e.data_ptr(), (PAIR_Q if side == "q" else 0)


def quantize(x: torch.Tensor, offsets=(-2, 6), hadamard: bool = False,
             global_scale: torch.Tensor | None = None, block: int = 16, workspace=None,
             signs=None, out=None, balance=None):
    """ScaleSearch NVFP4 quantize of x (last dim in blocks of 16).

    Returns (codes uint8[..., K/2], scales uint8[..., K/16], global_scale float32[1]).
    If ``global_scale`` (a device float32[1]) is given it is used as S_g.
    ``signs`` (four uint32 words) selects the randomized Hadamard transform.
    ``out`` = (codes, scales, global_scale) tensors to write instead of new ones
    (the third is ignored when ``global_scale`` is given).
    ``balance`` = (channel exponents, "q" or "k"): one side of the balancing pair
    (x 2^-e for Q, x 2^e for K; see ``balance_exponents``) before anything else.
    """
    L = load()
    dev = _dev(x)
    K = x.shape[-1]
    R = x.numel() // K if K else 0
    f_lo, f_hi = _offsets(offsets)
    flags = HADAMARD128 if hadamard else 0
    if out is not None:
        codes = _expect(out[0], "out codes", (*x.shape[:-1], K // 2), torch.uint8, dev)
        scales = _expect(out[1], "out scales", (*x.shape[:-1], K // 16), torch.uint8, dev)
    else:
        codes = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(*x.shape[:-1], K // 16, dtype=torch.uint8, device=dev)
    if global_scale is not None:
        flags |= GSCALE_GIVEN
        g = _scale_arg(global_scale, "global_scale", dev)
    elif out is not None:
        g = _scale_arg(out[2], "out global_scale", dev)
    else:
        g = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace, int(L.nvfp4_workspace_bytes(R, K, flags)), dev)
    sw = _signs(signs)
    if balance is not None:
        ep, pf = _balance(balance, K, dev)
        if sw is not None:
            flags |= HADAMARD128
        st = L.nvfp4_quantize_balanced(x.data_ptr(), _dtype(x), R, K, block, f_lo, f_hi,
                                       flags | pf, ep,
                                       None if sw is None else ctypes.addressof(sw),
                                       codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
                                       ws.data_ptr(), wsb, _stream(dev))
    elif sw is None:
        st = L.nvfp4_quantize(x.data_ptr(), _dtype(x), R, K, block, f_lo, f_hi, flags,
                              codes.data_ptr(), scales.data_ptr(), g.data_ptr(), ws.data_ptr(),
                              wsb, _stream(dev))
    else:
        st = L.nvfp4_quantize_rht(x.data_ptr(), _dtype(x), R, K, block, f_lo, f_hi, flags,
                                  ctypes.addressof(sw), codes.data_ptr(), scales.data_ptr(),
                                  g.data_ptr(), ws.data_ptr(), wsb, _stream(dev))
    _check("nvfp4_quantize", st)
    return codes, scales, g


def quantize_noalloc(x: torch.Tensor, offsets=(-2, 6), hadamard: bool = False,
                     global_scale: torch.Tensor | None = None, out=None):
    """``quantize`` through nvfp4_quantize_noalloc: the library keeps the amax pass's
    partial maxima in its own device array (no workspace). Calls that overlap in time on
    one GPU share that array and race. ``out`` = (codes, scales, global_scale) to write
    instead of new tensors (the third is ignored when ``global_scale`` is given)."""
    L = load()
    dev = _dev(x)
    K = x.shape[-1]
    R = x.numel() // K if K else 0
    f_lo, f_hi = _offsets(offsets)
    flags = HADAMARD128 if hadamard else 0
    if out is not None:
        codes = _expect(out[0], "out codes", (*x.shape[:-1], K // 2), torch.uint8, dev)
        scales = _expect(out[1], "out scales", (*x.shape[:-1], K // 16), torch.uint8, dev)
    else:
        codes = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8, device=dev)
        scales = torch.empty(*x.shape[:-1], K // 16, dtype=torch.uint8, device=dev)
    if global_scale is not None:
        flags |= GSCALE_GIVEN
        g = _scale_arg(global_scale, "global_scale", dev)
    elif out is not None:
        g = _scale_arg(out[2], "out global_scale", dev)
    else:
        g = torch.empty(1, dtype=torch.float32, device=dev)
    st = L.nvfp4_quantize_noalloc(x.data_ptr(), _dtype(x), R, K, 16, f_lo, f_hi, flags,
                                  codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
                                  _stream(dev))
    _check("nvfp4_quantize_noalloc", st)
    return codes, scales, g


def global_scale(x: torch.Tensor, hadamard: bool = False, workspace=None,
                 signs=None) -> torch.Tensor:
    """Tensor scale S_g = fl(max|x| / 2688) (1 if that is 0) as a device float32[1]."""
    L = load()
    dev = _dev(x)
    K = x.shape[-1]
    R = x.numel() // K if K else 0
    flags = HADAMARD128 if hadamard else 0
    g = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace, int(L.nvfp4_workspace_bytes(R, K, flags)), dev)
    sw = _signs(signs)
    if sw is None:
        st = L.nvfp4_global_scale(x.data_ptr(), _dtype(x), R, K, flags, g.data_ptr(),
                                  ws.data_ptr(), wsb, _stream(dev))
    else:
        st = L.nvfp4_global_scale_rht(x.data_ptr(), _dtype(x), R, K, flags, ctypes.addressof(sw),
                                      g.data_ptr(), ws.data_ptr(), wsb, _stream(dev))
    _check("nvfp4_global_scale", st)
    return g


def dequantize(codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor,
               out_dtype=torch.float32, block: int = 16, out: torch.Tensor | None = None):
    L = load()
    dev = _dev(codes)
    _expect(codes, "codes", None, torch.uint8, dev)
    K = codes.shape[-1] * 2
    R = codes.numel() * 2 // K if K else 0
    _expect(scales, "scales", (*codes.shape[:-1], K // 16), torch.uint8, dev)
    _scale_arg(global_scale, "global_scale", dev)
    if out is not None:
        y = _expect(out, "out", (*codes.shape[:-1], K), None, dev)
    else:
        y = torch.empty(*codes.shape[:-1], K, dtype=out_dtype, device=dev)
    st = L.nvfp4_dequantize(codes.data_ptr(), scales.data_ptr(), global_scale.data_ptr(), R, K,
                            block, y.data_ptr(), _dtype(y), _stream(dev))
    _check("nvfp4_dequantize", st)
    return y


def quantize_kv_sink(kv: torch.Tensor, n_first: int = 128, n_last: int = 128, offsets=(-2, 6),
                     hadamard: bool = False, global_scale: torch.Tensor | None = None,
                     block: int = 16, workspace=None, signs=None):
    """Attention-sink KV mode on kv[B, H, T, D].

    Returns (codes[B,H,Tm,D/2], scales[B,H,Tm,D/16], global_scale[1], sink[B,H,nf+nl,D]).
    """
    L = load()
    dev = _dev(kv)
    if kv.dim() != 4:
        raise ValueError("kv must be [B, H, T, D]")
    B, H, T, D = kv.shape
    Tm = T - n_first - n_last
    if Tm < 0 or n_first < 0 or n_last < 0:
        raise ValueError("n_first + n_last must not exceed T")
    f_lo, f_hi = _offsets(offsets)
    flags = HADAMARD128 if hadamard else 0
    codes = torch.empty(B, H, Tm, D // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(B, H, Tm, D // 16, dtype=torch.uint8, device=dev)
    sink = torch.empty(B, H, n_first + n_last, D, dtype=kv.dtype, device=dev)
    if global_scale is not None:
        flags |= GSCALE_GIVEN
        g = _scale_arg(global_scale, "global_scale", dev)
    else:
        g = torch.empty(1, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(workspace, int(L.nvfp4_workspace_bytes(B * H * Tm, D, flags)), dev)
    sw = _signs(signs)
    if sw is None:
        st = L.nvfp4_quantize_kv_sink(kv.data_ptr(), _dtype(kv), B, H, T, D, n_first, n_last,
                                      block, f_lo, f_hi, flags, codes.data_ptr(),
                                      scales.data_ptr(), g.data_ptr(), sink.data_ptr(),
                                      ws.data_ptr(), wsb, _stream(dev))
    else:
        st = L.nvfp4_quantize_kv_sink_rht(kv.data_ptr(), _dtype(kv), B, H, T, D, n_first, n_last,
                                          block, f_lo, f_hi, flags, ctypes.addressof(sw),
                                          codes.data_ptr(), scales.data_ptr(), g.data_ptr(),
                                          sink.data_ptr(), ws.data_ptr(), wsb, _stream(dev))
    _check("nvfp4_quantize_kv_sink", st)
    return codes, scales, g, sink


def dequantize_kv_sink(codes, scales, global_scale, sink, T: int, n_first: int, n_last: int,
                       out_dtype=torch.float32, block: int = 16):
    L = load()
    dev = _dev(codes)
    _dev(sink)
    if sink.dim() != 4:
        raise ValueError("sink must be [B, H, n_first + n_last, D]")
    B, H, NS, D = sink.shape
    if NS != n_first + n_last or T < NS:
        raise ValueError("sink holds n_first + n_last tokens, at most T")
    Tm = T - NS
    _expect(codes, "codes", (B, H, Tm, D // 2), torch.uint8, dev)
    _expect(scales, "scales", (B, H, Tm, D // 16), torch.uint8, dev)
    _scale_arg(global_scale, "global_scale", dev)
    y = torch.empty(B, H, T, D, dtype=out_dtype, device=dev)
    st = L.nvfp4_dequantize_kv_sink(codes.data_ptr(), scales.data_ptr(), global_scale.data_ptr(),
                                    sink.data_ptr(), _dtype(sink), B, H, T, D, n_first, n_last,
                                    block, y.data_ptr(), _dtype(y), _stream(dev))
    _check("nvfp4_dequantize_kv_sink", st)
    return y


def hadamard128(x: torch.Tensor, signs=None, balance=None) -> torch.Tensor:
    """FP32 y = x H / sqrt(128) per 128-vector (x bf16), as the quantizer computes it;
    with ``signs``, y = (x o s) H / sqrt(128); with ``balance`` = (exponents, side)
    (x[..., 128] only), x is first scaled by 2^-e (side "q") or 2^e ("k")."""
    L = load()
    dev = _dev(x)
    if x.shape[-1] % 128:
        raise ValueError("last dimension must be a multiple of 128")
    y = torch.empty(x.shape, dtype=torch.float32, device=dev)
    sw = _signs(signs)
    if balance is not None:
        if x.shape[-1] != 128:
            raise ValueError("the balancing pair with the transform needs a last dimension of 128")
        ep, pf = _balance(balance, 128, dev)
        st = L.nvfp4_hadamard128_balanced(x.data_ptr(), _dtype(x), x.numel() // 128, ep, pf,
                                          None if sw is None else ctypes.addressof(sw),
                                          y.data_ptr(), _stream(dev))
    elif sw is None:
        st = L.nvfp4_hadamard128(x.data_ptr(), _dtype(x), x.numel() // 128, y.data_ptr(),
                                 _stream(dev))
    else:
        st = L.nvfp4_hadamard128_rht(x.data_ptr(), _dtype(x), x.numel() // 128,
                                     ctypes.addressof(sw), y.data_ptr(), _stream(dev))
    _check("nvfp4_hadamard128", st)
    return y


def balance_exponents(q: torch.Tensor, k: torch.Tensor, workspace=None) -> torch.Tensor:
    """Channel exponents (device int8 [D]) of the balancing pair Q' = Q 2^-e, K' = K 2^e
    from calibration tensors q [..., D] and k [..., D] (same dtype, D % 16 == 0,
    D <= 2048): per channel the integer e minimising its share of ||Q'||^2 + ||K'||^2."""
    L = load()
    dev = _dev(q)
    _expect(k, "k", None, q.dtype, dev)
    D = q.shape[-1]
    if k.shape[-1] != D:
        raise ValueError("q and k must have the same last dimension")
    e = torch.empty(D, dtype=torch.int8, device=dev)
    ws, wsb = _workspace(workspace, int(L.nvfp4_balance_workspace_bytes(D)), dev)
    st = L.nvfp4_balance_exponents(q.data_ptr(), k.data_ptr(), _dtype(q), q.numel() // D,
                                   k.numel() // D, D, e.data_ptr(), ws.data_ptr(), wsb,
                                   _stream(dev))
    _check("nvfp4_balance_exponents", st)
    return e


def kv_cache_alloc(B: int, H: int, D: int, capacity: int, n_first: int = 128, n_last: int = 128,
                   dtype=torch.bfloat16, device="cuda"):
    """Buffers of an attention-sink NVFP4 KV cache for up to `capacity` tokens per (b, h):
    head [B, H, n_first, D], tail ring [B, H, n_last, D], codes [B, H, cap, D/2],
    scales [B, H, cap, D/16] with cap = capacity - n_first - n_last middle rows; the
    token count as a host int ("length", kv_append) and as a device int64[1]
    ("length_dev", kv_append_dev and attention_kv_cache_dev)."""
    cap = max(capacity - n_first - n_last, 0)
    return dict(
        head=torch.empty(B, H, n_first, D, dtype=dtype, device=device),
        tail=torch.empty(B, H, n_last, D, dtype=dtype, device=device),
        codes=torch.empty(B, H, cap, D // 2, dtype=torch.uint8, device=device),
        scales=torch.empty(B, H, cap, D // 16, dtype=torch.uint8, device=device),
        length_dev=torch.zeros(1, dtype=torch.int64, device=device),
        n_first=n_first, n_last=n_last, length=0)


def _cache_args(cache: dict, kv_new: torch.Tensor, global_scale: torch.Tensor):
    dev = _dev(kv_new)
    _scale_arg(global_scale, "global_scale", dev)
    if kv_new.dim() != 4:
        raise ValueError("kv_new must be [B, H, t_new, D]")
    B, H, t_new, D = kv_new.shape
    nf, nl = cache["n_first"], cache["n_last"]
    cap = cache["codes"].shape[2] if cache["codes"].dim() == 4 else -1
    head = _expect(cache["head"], "cache head", (B, H, nf, D), kv_new.dtype, dev)
    tail = _expect(cache["tail"], "cache tail", (B, H, nl, D), kv_new.dtype, dev)
    codes = _expect(cache["codes"], "cache codes", (B, H, cap, D // 2), torch.uint8, dev)
    scales = _expect(cache["scales"], "cache scales", (B, H, cap, D // 16), torch.uint8, dev)
    return dev, B, H, t_new, D, nf, nl, cap, head, tail, codes, scales


def kv_append_dev(cache: dict, kv_new: torch.Tensor, global_scale: torch.Tensor, offsets=(-2, 6),
                  hadamard: bool = False, block: int = 16, signs=None):
    """kv_append at the device-resident length cache["length_dev"] (read and advanced on
    the device, so the call can be captured in a HIP graph and replayed per token; an
    append that would not fit leaves cache and length unchanged). cache["length"] (the
    host count) is not touched; kv_length reads the device one."""
    L = load()
    dev, B, H, t_new, D, nf, nl, cap, head, tail, codes, scales = _cache_args(cache, kv_new,
                                                                             global_scale)
    length = _expect(cache["length_dev"], "cache length_dev", (1,), torch.int64, dev)
    f_lo, f_hi = _offsets(offsets)
    flags = HADAMARD128 if hadamard else 0
    sw = _signs(signs)
    st = L.nvfp4_kv_append_dev(kv_new.data_ptr(), _dtype(kv_new), B, H, t_new, D, nf, nl, cap,
                               block, f_lo, f_hi, flags,
                               ctypes.addressof(sw) if sw is not None else None,
                               global_scale.data_ptr(), head.data_ptr(), tail.data_ptr(),
                               codes.data_ptr(), scales.data_ptr(), length.data_ptr(),
                               _stream(dev))
    _check("nvfp4_kv_append_dev", st)
    return cache


class _KvCacheRef(ctypes.Structure):
    """nvfp4_kv_cache_ref: one cache of nvfp4_kv_append2_dev."""
    _fields_ = [("kv_new", _vp), ("flags", _u32), ("signs", _vp), ("global_scale", _vp),
                ("head", _vp), ("tail", _vp), ("codes", _vp), ("scales", _vp), ("length", _vp)]


def kv_append2_dev(k_cache: dict, k_new: torch.Tensor, k_gscale: torch.Tensor, v_cache: dict,
                   v_new: torch.Tensor, v_gscale: torch.Tensor, offsets=(-2, 6),
                   k_hadamard: bool = False, v_hadamard: bool = False, k_signs=None,
                   v_signs=None, block: int = 16):
    """kv_append_dev on k_cache, then on v_cache, in one call: a decode step's two
    appends (small, no Hadamard) run as one launch. Both caches hold the same
    geometry and each its own device-resident length."""
    L = load()
    refs, keep, geo = [], [], []
    for cache, new, gs, had, signs in ((k_cache, k_new, k_gscale, k_hadamard, k_signs),
                                       (v_cache, v_new, v_gscale, v_hadamard, v_signs)):
        dev, B, H, t_new, D, nf, nl, cap, head, tail, codes, scales = _cache_args(cache, new, gs)
        length = _expect(cache["length_dev"], "cache length_dev", (1,), torch.int64, dev)
        sw = _signs(signs)
        keep.append(sw)
        refs.append(_KvCacheRef(new.data_ptr(), HADAMARD128 if had else 0,
                                ctypes.addressof(sw) if sw is not None else None, gs.data_ptr(),
                                head.data_ptr(), tail.data_ptr(), codes.data_ptr(),
                                scales.data_ptr(), length.data_ptr()))
        geo.append((dev, B, H, t_new, D, nf, nl, cap, _dtype(new)))
    if geo[0] != geo[1]:
        raise ValueError(f"kv_append2_dev: K and V differ in device, shape or dtype: {geo}")
    dev, B, H, t_new, D, nf, nl, cap, dt = geo[0]
    f_lo, f_hi = _offsets(offsets)
    st = L.nvfp4_kv_append2_dev(ctypes.addressof(refs[0]), ctypes.addressof(refs[1]), dt, B, H,
                                t_new, D, nf, nl, cap, block, f_lo, f_hi, _stream(dev))
    _check("nvfp4_kv_append2_dev", st)
    return k_cache, v_cache


def kv_length(cache: dict) -> int:
    """The device-resident token count of a cache (synchronizes with the device)."""
    return int(cache["length_dev"].item())


def kv_append(cache: dict, kv_new: torch.Tensor, global_scale: torch.Tensor, offsets=(-2, 6),
              hadamard: bool = False, block: int = 16, signs=None):
    """Append kv_new [B, H, t_new, D] to a cache made by kv_cache_alloc (in place)."""
    L = load()
    dev, B, H, t_new, D, nf, nl, cap, head, tail, codes, scales = _cache_args(cache, kv_new,
                                                                             global_scale)
    f_lo, f_hi = _offsets(offsets)
    flags = HADAMARD128 if hadamard else 0
    T = cache["length"]
    sw = _signs(signs)
    if sw is None:
        st = L.nvfp4_kv_append(kv_new.data_ptr(), _dtype(kv_new), B, H, T, t_new, D,
                               cache["n_first"], cache["n_last"], codes.shape[2], block, f_lo,
                               f_hi, flags, global_scale.data_ptr(), head.data_ptr(),
                               tail.data_ptr(), codes.data_ptr(), scales.data_ptr(), _stream(dev))
    else:
        st = L.nvfp4_kv_append_rht(kv_new.data_ptr(), _dtype(kv_new), B, H, T, t_new, D,
                                   cache["n_first"], cache["n_last"], codes.shape[2], block, f_lo,
                                   f_hi, flags, ctypes.addressof(sw), global_scale.data_ptr(),
                                   head.data_ptr(), tail.data_ptr(), codes.data_ptr(),
                                   scales.data_ptr(), _stream(dev))
    _check("nvfp4_kv_append", st)
    cache["length"] = T + t_new
    return cache


def mxfp4_quantize(x: torch.Tensor, offsets=(0, 0), block: int = 32):
    """MXFP4 (32-element blocks, E8M0 power-of-two scales) of x: returns
    (codes uint8[..., K/2], scales uint8[..., K/32]); offsets search the exponent."""
    L = load()
    dev = _dev(x)
    K = x.shape[-1]
    R = x.numel() // K if K else 0
    f_lo, f_hi = _offsets(offsets)
    codes = torch.empty(*x.shape[:-1], K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(*x.shape[:-1], K // 32, dtype=torch.uint8, device=dev)
    st = L.mxfp4_quantize(x.data_ptr(), _dtype(x), R, K, block, f_lo, f_hi, codes.data_ptr(),
                          scales.data_ptr(), _stream(dev))
    _check("mxfp4_quantize", st)
    return codes, scales


def mxfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, out_dtype=torch.float32,
                     block: int = 32, out: torch.Tensor | None = None):
    L = load()
    dev = _dev(codes)
    _expect(codes, "codes", None, torch.uint8, dev)
    K = codes.shape[-1] * 2
    R = codes.numel() * 2 // K if K else 0
    _expect(scales, "scales", (*codes.shape[:-1], K // 32), torch.uint8, dev)
    if out is not None:
        y = _expect(out, "out", (*codes.shape[:-1], K), None, dev)
    else:
        y = torch.empty(*codes.shape[:-1], K, dtype=out_dtype, device=dev)
    st = L.mxfp4_dequantize(codes.data_ptr(), scales.data_ptr(), R, K, block, y.data_ptr(),
                            _dtype(y), _stream(dev))
    _check("mxfp4_dequantize", st)
    return y


def attention(q, k, v, causal: bool = False, out_dtype=torch.float32):
    """Attention on NVFP4 operands. q, k, v: (codes [B, H, N, 64], scales [B, H, N, 8],
    global_scale float32[1]) as ``quantize`` returns them for [B, H, N, 128] tensors;
    k and v may have fewer heads than q. Returns O [B, Hq, Nq, 128]."""
    L = load()
    qc, qs, qg = q
    kc, ks, kg = k
    vc, vs, vg = v
    dev = _dev(qc)
    if qc.dim() != 4 or kc.dim() != 4 or vc.shape != kc.shape:
        raise ValueError("q, k, v codes must be [B, H, N, 64] with matching k and v")
    B, Hq, Nq, D2 = qc.shape
    Hkv, Nk = kc.shape[1], kc.shape[2]
    _expect(qc, "q codes", None, torch.uint8, dev)
    _expect(qs, "q scales", (B, Hq, Nq, D2 // 8), torch.uint8, dev)
    for name, c, sc in (("k", kc, ks), ("v", vc, vs)):
        _expect(c, f"{name} codes", (B, Hkv, Nk, D2), torch.uint8, dev)
        _expect(sc, f"{name} scales", (B, Hkv, Nk, D2 // 8), torch.uint8, dev)
    for name, g in (("q", qg), ("k", kg), ("v", vg)):
        _scale_arg(g, f"{name} global_scale", dev)
    y = torch.empty(B, Hq, Nq, D2 * 2, dtype=out_dtype, device=dev)
    st = L.nvfp4_attention(qc.data_ptr(), qs.data_ptr(), qg.data_ptr(), kc.data_ptr(),
                           ks.data_ptr(), kg.data_ptr(), vc.data_ptr(), vs.data_ptr(),
                           vg.data_ptr(), B, Hq, Hkv, Nq, Nk, D2 * 2, int(causal), y.data_ptr(),
                           _dtype(y), _stream(dev))
    _check("nvfp4_attention", st)
    return y


def attention_split_workspace_bytes(B: int, Hq: int, Nq: int, cap: int, split: int) -> int:
    """Workspace bytes of attention_kv_cache(..., split=split) for a cache of `cap`
    middle rows (0 if the split calls would reject these sizes)."""
    return int(load().nvfp4_attention_split_workspace_bytes(B, Hq, Nq, cap, split))


def attention_kv_cache(q, k_cache: dict, k_gscale: torch.Tensor, v_cache: dict,
                       v_gscale: torch.Tensor, out_dtype=torch.float32, device_length: bool = False,
                       split: int = 0, workspace: torch.Tensor | None = None):
    """Attention of q (codes, scales, global_scale of [B, Hq, Nq, 128]) over K and V
    sink caches made by kv_cache_alloc and filled by kv_append (bf16). Returns O.
    With device_length, the token count is k_cache["length_dev"], read on the device
    (for caches filled by kv_append_dev; capturable in a HIP graph). split > 0 (a
    multiple of 32): the head, the tail and each piece of `split` middle tokens run
    on their own workgroups and are merged (for decode steps with few queries);
    workspace: a device tensor of attention_split_workspace_bytes bytes, else one
    is allocated."""
    L = load()
    qc, qs, qg = q
    dev = _dev(qc)
    if qc.dim() != 4 or k_cache["codes"].dim() != 4:
        raise ValueError("q codes must be [B, Hq, Nq, 64]; cache codes [B, Hkv, cap, 64]")
    if (k_cache["n_first"], k_cache["n_last"], k_cache["codes"].shape) != \
            (v_cache["n_first"], v_cache["n_last"], v_cache["codes"].shape):
        raise ValueError("the K and V caches have different layouts")
    if not device_length and k_cache["length"] != v_cache["length"]:
        raise ValueError("the K and V caches hold different numbers of tokens")
    B, Hq, Nq, D2 = qc.shape
    Hkv, cap = k_cache["codes"].shape[1], k_cache["codes"].shape[2]
    nf, nl, D = k_cache["n_first"], k_cache["n_last"], 2 * D2
    _expect(qc, "q codes", None, torch.uint8, dev)
    _expect(qs, "q scales", (B, Hq, Nq, D2 // 8), torch.uint8, dev)
    for name, g in (("q", qg), ("k", k_gscale), ("v", v_gscale)):
        _scale_arg(g, f"{name} global_scale", dev)
    for which, c in (("k", k_cache), ("v", v_cache)):
        _expect(c["head"], f"{which} cache head", (B, Hkv, nf, D), torch.bfloat16, dev)
        _expect(c["tail"], f"{which} cache tail", (B, Hkv, nl, D), torch.bfloat16, dev)
        _expect(c["codes"], f"{which} cache codes", (B, Hkv, cap, D2), torch.uint8, dev)
        _expect(c["scales"], f"{which} cache scales", (B, Hkv, cap, D2 // 8), torch.uint8, dev)
    y = torch.empty(B, Hq, Nq, D2 * 2, dtype=out_dtype, device=dev)
    ptrs = (qc.data_ptr(), qs.data_ptr(), qg.data_ptr(), k_cache["head"].data_ptr(),
            k_cache["tail"].data_ptr(), k_cache["codes"].data_ptr(), k_cache["scales"].data_ptr(),
            k_gscale.data_ptr(), v_cache["head"].data_ptr(), v_cache["tail"].data_ptr(),
            v_cache["codes"].data_ptr(), v_cache["scales"].data_ptr(), v_gscale.data_ptr())
    if device_length:
        length = _expect(k_cache["length_dev"], "cache length_dev", (1,), torch.int64, dev)
        tokens, fn = length.data_ptr(), "nvfp4_attention_kv_cache_dev"
    else:
        tokens, fn = k_cache["length"], "nvfp4_attention_kv_cache"
    if split:
        ws, nbytes = _workspace(workspace, attention_split_workspace_bytes(B, Hq, Nq, cap, split),
                                dev)
        fn = fn.replace("kv_cache", "kv_cache_split")
        st = getattr(L, fn)(*ptrs, BF16, B, Hq, Hkv, Nq, tokens, D, nf, nl, cap, split,
                            ws.data_ptr(), nbytes, y.data_ptr(), _dtype(y), _stream(dev))
    else:
        st = getattr(L, fn)(*ptrs, BF16, B, Hq, Hkv, Nq, tokens, D, nf, nl, cap, y.data_ptr(),
                            _dtype(y), _stream(dev))
    _check(fn, st)
    return y
