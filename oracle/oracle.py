"""ctypes binding of the C oracle (``nvfp4_oracle.c``).

TEST INFRASTRUCTURE (see the package docstring). Host NumPy arrays only:
FP32 tensors are ``float32`` arrays and bf16 tensors are ``uint16`` arrays
holding the bfloat16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# The oracle is compiled with plain gcc: IEEE binary32 on x86-64 SSE, no
# contraction of a*b+c into FMA, no fast-math.
GCC_CMD = [
    "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
    "-fno-fast-math", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB, "-lm",
]

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle library (``force=False``: only if it is missing)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = GCC_CMD[:-3] + ["-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
            vp = ctypes.c_void_p
            L.oracle_e2m1_code.argtypes = [f32]
            L.oracle_e2m1_code.restype = i32
            L.oracle_e4m3_value.argtypes = [i32]
            L.oracle_e4m3_value.restype = f32
            L.oracle_e4m3_encode.argtypes = [f32]
            L.oracle_e4m3_encode.restype = i32
            L.oracle_e2m1_code_batch.argtypes = [vp, i64, vp]
            L.oracle_e2m1_code_batch.restype = None
            L.oracle_e4m3_encode_batch.argtypes = [vp, i64, vp]
            L.oracle_e4m3_encode_batch.restype = None
            L.oracle_block_sse.argtypes = [vp, f32, i32]
            L.oracle_block_sse.restype = f32
            L.oracle_quantize.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, i32]
            L.oracle_quantize.restype = i32
            L.oracle_dequantize.argtypes = [vp, vp, f32, i64, i64, i32, vp]
            L.oracle_dequantize.restype = i32
            L.oracle_quantize_kv_sink.argtypes = [vp, i32, i64, i64, i64, i64, i64, i64, i32, i32,
                                                  i32, i32, vp, vp, vp, vp, i32]
            L.oracle_quantize_kv_sink.restype = i32
            L.oracle_dequantize_kv_sink.argtypes = [vp, vp, f32, vp, i32, i64, i64, i64, i64, i64,
                                                    i64, i32, vp]
            L.oracle_dequantize_kv_sink.restype = i32
            L.oracle_hadamard128.argtypes = [vp, i32, i64, vp, i32]
            L.oracle_hadamard128.restype = i32
            L.oracle_hadamard128_rht.argtypes = [vp, i32, i64, vp, vp, i32]
            L.oracle_hadamard128_rht.restype = i32
            L.oracle_quantize_rht.argtypes = [vp, i32, i64, i64, vp, i32, i32, i32, vp, vp, vp, i32]
            L.oracle_quantize_rht.restype = i32
            L.oracle_balance_exponent.argtypes = [ctypes.c_double, ctypes.c_double]
            L.oracle_balance_exponent.restype = i32
            L.oracle_balance_exponents.argtypes = [vp, vp, i32, i64, i64, i64, vp]
            L.oracle_balance_exponents.restype = i32
            L.oracle_quantize_balanced.argtypes = [vp, i32, i64, i64, vp, i32, i32, vp, i32, i32,
                                                   i32, vp, vp, vp, i32]
            L.oracle_quantize_balanced.restype = i32
            L.oracle_hadamard128_balanced.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, i32]
            L.oracle_hadamard128_balanced.restype = i32
            L.oracle_quantize_mxfp4.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, i32]
            L.oracle_quantize_mxfp4.restype = i32
            L.oracle_dequantize_mxfp4.argtypes = [vp, vp, i64, i64, i32, vp]
            L.oracle_dequantize_mxfp4.restype = i32
            L.oracle_mx_block_sse.argtypes = [vp, i32]
            L.oracle_mx_block_sse.restype = f32
            L.oracle_attention_nvfp4.argtypes = [vp, vp, f32, vp, vp, f32, vp, vp, f32, i64, i64,
                                                 i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp,
                                                 vp, vp, i32]
            L.oracle_attention_nvfp4.restype = i32
            L.oracle_attention_kv_cache.argtypes = [vp, vp, f32, vp, vp, vp, vp, f32, vp, vp, vp,
                                                    vp, f32, i64, i64, i64, i64, i64, i64, i64,
                                                    i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                                    vp, i32]
            L.oracle_attention_kv_cache.restype = i32
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits)")


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


def e2m1_code(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.int8)
    lib().oracle_e2m1_code_batch(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.int16)
    lib().oracle_e4m3_encode_batch(_ptr(t), t.size, _ptr(out))
    return out


def e4m3_value(p: int) -> float:
    return float(lib().oracle_e4m3_value(int(p)))


def block_sse(x16, sg: float, p: int) -> float:
    x = np.ascontiguousarray(x16, dtype=np.float32).reshape(16)
    return float(np.float32(lib().oracle_block_sse(_ptr(x), ctypes.c_float(sg), int(p))))


def quantize(x: np.ndarray, f_lo: int = -2, f_hi: int = 6, hadamard: bool = False,
             gscale: float | None = None, want_f: bool = False, nthreads: int | None = None):
    """Returns (codes[R, K/2] u8, scales[R, K/16] u8, gscale f32[, chosen_f[R, K/16] i8])."""
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    K = x.shape[-1]
    R = x.size // K if K else 0
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 16), dtype=np.uint8)
    g = np.array([0.0 if gscale is None else gscale], dtype=np.float32)
    fsel = np.empty((R, K // 16), dtype=np.int8) if want_f else None
    rc = lib().oracle_quantize(_ptr(x), dt, R, K, f_lo, f_hi, int(hadamard),
                               int(gscale is not None), _ptr(g), _ptr(codes), _ptr(scales),
                               _ptr(fsel) if want_f else None, _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_quantize failed ({rc})")
    shp = x.shape[:-1]
    out = (codes.reshape(*shp, K // 2), scales.reshape(*shp, K // 16), np.float32(g[0]))
    if want_f:
        return out + (fsel.reshape(*shp, K // 16),)
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, gscale: float, out: str = "f32"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = codes.shape[-1] * 2
    R = codes.size * 2 // K if K else 0
    odt = F32 if out == "f32" else BF16
    y = np.empty(codes.shape[:-1] + (K,), dtype=np.float32 if odt == F32 else np.uint16)
    rc = lib().oracle_dequantize(_ptr(codes), _ptr(scales), ctypes.c_float(gscale), R, K, odt,
                                 _ptr(y))
    if rc:
        raise ValueError(f"oracle_dequantize failed ({rc})")
    return y


def quantize_kv_sink(kv: np.ndarray, n_first: int, n_last: int, f_lo: int = -2, f_hi: int = 6,
                     hadamard: bool = False, gscale: float | None = None,
                     nthreads: int | None = None):
    """kv [B, H, T, D] -> (codes[B,H,Tm,D/2], scales[B,H,Tm,D/16], gscale, sink[B,H,nf+nl,D])."""
    kv = np.ascontiguousarray(kv)
    dt = _dtype_of(kv)
    B, H, T, D = kv.shape
    Tm = T - n_first - n_last
    codes = np.empty((B, H, Tm, D // 2), dtype=np.uint8)
    scales = np.empty((B, H, Tm, D // 16), dtype=np.uint8)
    sink = np.empty((B, H, n_first + n_last, D), dtype=kv.dtype)
    g = np.array([0.0 if gscale is None else gscale], dtype=np.float32)
    rc = lib().oracle_quantize_kv_sink(_ptr(kv), dt, B, H, T, D, n_first, n_last, f_lo, f_hi,
                                       int(hadamard), int(gscale is not None), _ptr(g),
                                       _ptr(codes), _ptr(scales), _ptr(sink), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_quantize_kv_sink failed ({rc})")
    return codes, scales, np.float32(g[0]), sink


def dequantize_kv_sink(codes, scales, gscale, sink, T: int, n_first: int, n_last: int,
                       out: str = "f32"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    sink = np.ascontiguousarray(sink)
    B, H, _, D = sink.shape
    odt = F32 if out == "f32" else BF16
    y = np.empty((B, H, T, D), dtype=np.float32 if odt == F32 else np.uint16)
    rc = lib().oracle_dequantize_kv_sink(_ptr(codes), _ptr(scales), ctypes.c_float(gscale),
                                         _ptr(sink), _dtype_of(sink), B, H, T, D, n_first,
                                         n_last, odt, _ptr(y))
    if rc:
        raise ValueError(f"oracle_dequantize_kv_sink failed ({rc})")
    return y


def hadamard128(x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    if x.shape[-1] % 128:
        raise ValueError("last dimension must be a multiple of 128")
    y = np.empty(x.shape, dtype=np.float32)
    rc = lib().oracle_hadamard128(_ptr(x), dt, x.size // 128, _ptr(y), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_hadamard128 failed ({rc})")
    return y


def _signs_words(signs) -> np.ndarray:
    """128 sign bits as four uint32 words (bit k of word k // 32: negate feature k)."""
    w = np.ascontiguousarray(signs, dtype=np.uint32)
    if w.shape != (4,):
        raise ValueError("signs: four uint32 words")
    return w


def hadamard128_rht(x: np.ndarray, signs, nthreads: int | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    w = _signs_words(signs)
    y = np.empty(x.shape, dtype=np.float32)
    rc = lib().oracle_hadamard128_rht(_ptr(x), dt, x.size // 128, _ptr(w), _ptr(y),
                                      _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_hadamard128_rht failed ({rc})")
    return y


def quantize_rht(x: np.ndarray, signs, f_lo: int = -8, f_hi: int = 8, gscale: float | None = None,
                 nthreads: int | None = None):
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    w = _signs_words(signs)
    K = x.shape[-1]
    R = x.size // K
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 16), dtype=np.uint8)
    g = np.array([0.0 if gscale is None else gscale], dtype=np.float32)
    rc = lib().oracle_quantize_rht(_ptr(x), dt, R, K, _ptr(w), f_lo, f_hi, int(gscale is not None),
                                   _ptr(g), _ptr(codes), _ptr(scales), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_quantize_rht failed ({rc})")
    shp = x.shape[:-1]
    return codes.reshape(*shp, K // 2), scales.reshape(*shp, K // 16), np.float32(g[0])


def balance_exponent(a2: float, b2: float) -> int:
    """The channel exponent of the balancing pair for sums of squares a2 (Q) and b2 (K)."""
    return int(lib().oracle_balance_exponent(float(a2), float(b2)))


def balance_exponents(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Channel exponents e (int8 [D]) of the balancing pair Q' = Q diag(2^-e),
    K' = K diag(2^e), from calibration tensors q [..., D] and k [..., D] (same dtype)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    dt = _dtype_of(q)
    if _dtype_of(k) != dt or q.shape[-1] != k.shape[-1]:
        raise ValueError("q and k: same dtype and last dimension")
    D = q.shape[-1]
    e = np.zeros(D, dtype=np.int8)
    rc = lib().oracle_balance_exponents(_ptr(q), _ptr(k), dt, q.size // D, k.size // D, D, _ptr(e))
    if rc:
        raise ValueError(f"oracle_balance_exponents failed ({rc})")
    return e


def quantize_balanced(x: np.ndarray, e, side: int, f_lo: int = -2, f_hi: int = 6,
                      hadamard: bool = False, signs=None, gscale: float | None = None,
                      nthreads: int | None = None):
    """Quantize one side of the balancing pair: x diag(2^(side e)) (side -1 for Q, +1
    for K), optionally followed by the (randomized, with signs) Hadamard transform."""
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    K = x.shape[-1]
    R = x.size // K
    e = np.ascontiguousarray(e, dtype=np.int8)
    if e.shape != (K,):
        raise ValueError("e: one exponent per column")
    w = None if signs is None else _signs_words(signs)
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 16), dtype=np.uint8)
    g = np.array([0.0 if gscale is None else gscale], dtype=np.float32)
    rc = lib().oracle_quantize_balanced(_ptr(x), dt, R, K, _ptr(e), int(side), int(hadamard),
                                        None if w is None else _ptr(w), f_lo, f_hi,
                                        int(gscale is not None), _ptr(g), _ptr(codes),
                                        _ptr(scales), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_quantize_balanced failed ({rc})")
    shp = x.shape[:-1]
    return codes.reshape(*shp, K // 2), scales.reshape(*shp, K // 16), np.float32(g[0])


def hadamard128_balanced(x: np.ndarray, e, side: int, signs=None,
                         nthreads: int | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    K = x.shape[-1]
    e = np.ascontiguousarray(e, dtype=np.int8)
    w = None if signs is None else _signs_words(signs)
    y = np.empty(x.shape, dtype=np.float32)
    rc = lib().oracle_hadamard128_balanced(_ptr(x), dt, x.size // K, K, _ptr(e), int(side),
                                           None if w is None else _ptr(w), _ptr(y),
                                           _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_hadamard128_balanced failed ({rc})")
    return y


def quantize_mxfp4(x: np.ndarray, f_lo: int = 0, f_hi: int = 0, nthreads: int | None = None):
    """MXFP4 (32-element blocks, E8M0 scales): (codes[R, K/2] u8, scales[R, K/32] u8)."""
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    K = x.shape[-1]
    R = x.size // K
    codes = np.empty((R, K // 2), dtype=np.uint8)
    scales = np.empty((R, K // 32), dtype=np.uint8)
    rc = lib().oracle_quantize_mxfp4(_ptr(x), dt, R, K, f_lo, f_hi, _ptr(codes), _ptr(scales),
                                     _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_quantize_mxfp4 failed ({rc})")
    shp = x.shape[:-1]
    return codes.reshape(*shp, K // 2), scales.reshape(*shp, K // 32)


def dequantize_mxfp4(codes: np.ndarray, scales: np.ndarray, out: str = "f32"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = codes.shape[-1] * 2
    R = codes.size * 2 // K
    odt = F32 if out == "f32" else BF16
    y = np.empty(codes.shape[:-1] + (K,), dtype=np.float32 if odt == F32 else np.uint16)
    rc = lib().oracle_dequantize_mxfp4(_ptr(codes), _ptr(scales), R, K, odt, _ptr(y))
    if rc:
        raise ValueError(f"oracle_dequantize_mxfp4 failed ({rc})")
    return y


def mx_block_sse(x32, X: int) -> float:
    x = np.ascontiguousarray(x32, dtype=np.float32).reshape(32)
    return float(np.float32(lib().oracle_mx_block_sse(_ptr(x), int(X))))


def _attention_terms(O, rs, us, mp, rowinfo):
    """The comparison terms the attention oracle returns beside O: per element rs (sum
    over tiles of |acc| at each tile's start), us (split keys: sum over units of
    |w_u acc_u|) and mp (magnitude sum of the keys whose P was coded against a running
    max other than the final one), all in units of O; per query row nres (tiles that
    may move the running max), ntiles (most tiles one softmax state visits), dmax
    (largest relative error allowance on a p) and units (softmax states merged)."""
    shp = O.shape[:-1]
    ri = rowinfo.reshape(*shp, 4)
    return {"rs": rs, "us": us, "mp": mp, "nres": ri[..., 0], "ntiles": ri[..., 1],
            "dmax": ri[..., 2], "units": ri[..., 3]}


def attention_nvfp4(q, k, v, tile: int = 32, causal: bool = False, nthreads: int | None = None,
                    terms: bool = False):
    """Attention on NVFP4 operands. q, k, v: (codes [B,H,N,D/2] u8, scales [B,H,N,D/16] u8,
    tensor scale); k and v may have fewer heads (shared by groups of query heads).
    Returns (O, mag, bound) as float64 [B, Hq, Nq, D], and with terms=True a fourth item,
    the dict of _attention_terms."""
    qc, qs, qg = q
    kc, ks, kg = k
    vc, vs, vg = v
    qc, qs, kc, ks, vc, vs = (np.ascontiguousarray(a, dtype=np.uint8)
                              for a in (qc, qs, kc, ks, vc, vs))
    B, Hq, Nq, D2 = qc.shape
    Hkv, Nk = kc.shape[1], kc.shape[2]
    D = D2 * 2
    O = np.zeros((B, Hq, Nq, D), np.float64)
    mag, bound, rs, us, mp = (np.zeros_like(O) for _ in range(5))
    rowinfo = np.zeros((B, Hq, Nq, 4), np.float64)
    rc = lib().oracle_attention_nvfp4(_ptr(qc), _ptr(qs), float(qg), _ptr(kc), _ptr(ks), float(kg),
                                      _ptr(vc), _ptr(vs), float(vg), B, Hq, Hkv, Nq, Nk, D, tile,
                                      int(causal), _ptr(O), _ptr(mag), _ptr(bound), _ptr(rs),
                                      _ptr(us), _ptr(mp), _ptr(rowinfo), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_attention_nvfp4 failed ({rc})")
    if terms:
        return O, mag, bound, _attention_terms(O, rs, us, mp, rowinfo)
    return O, mag, bound


def attention_kv_cache(q, k, v, T: int, n_first: int, n_last: int, tile: int = 32,
                       split: int = 0, nthreads: int | None = None, terms: bool = False):
    """Attention over the attention-sink KV cache. q: (codes, scales, tensor scale) of
    [B, Hq, Nq, D]; k, v: dicts with head [B,H,nf,D], tail [B,H,nl,D] (bf16 bits, ring by
    token mod nl), codes [B,H,cap,D/2], scales [B,H,cap,D/16], gscale. split > 0 (a
    multiple of tile): head, tail and each piece of `split` middle tokens run their
    softmax alone and are combined. Returns (O, mag, bound), and with terms=True the dict
    of _attention_terms as a fourth item."""
    qc, qs, qg = q
    qc = np.ascontiguousarray(qc, dtype=np.uint8)
    qs = np.ascontiguousarray(qs, dtype=np.uint8)
    B, Hq, Nq, D2 = qc.shape
    D = D2 * 2
    Hkv = k["codes"].shape[1]
    cap = k["codes"].shape[2]
    arr = lambda a, dt: np.ascontiguousarray(a, dtype=dt)
    kh, kt, vh, vt = (arr(x, np.uint16) for x in (k["head"], k["tail"], v["head"], v["tail"]))
    kc, ks, vc, vs = (arr(x, np.uint8) for x in (k["codes"], k["scales"], v["codes"], v["scales"]))
    O = np.zeros((B, Hq, Nq, D), np.float64)
    mag, bound, rs, us, mp = (np.zeros_like(O) for _ in range(5))
    rowinfo = np.zeros((B, Hq, Nq, 4), np.float64)
    rc = lib().oracle_attention_kv_cache(_ptr(qc), _ptr(qs), float(qg), _ptr(kh), _ptr(kt),
                                         _ptr(kc), _ptr(ks), float(k["gscale"]), _ptr(vh),
                                         _ptr(vt), _ptr(vc), _ptr(vs), float(v["gscale"]), B, Hq,
                                         Hkv, Nq, T, D, n_first, n_last, cap, tile, split,
                                         _ptr(O), _ptr(mag), _ptr(bound), _ptr(rs), _ptr(us),
                                         _ptr(mp), _ptr(rowinfo), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_attention_kv_cache failed ({rc})")
    if terms:
        return O, mag, bound, _attention_terms(O, rs, us, mp, rowinfo)
    return O, mag, bound
