"""The C-ABI library loads and exports every symbol include/*.h declares, and
rejects bad arguments on the host (no GPU needed: checks run before any launch)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    from microscaling_fp4_block_amd import build, nvfp4

    alt = os.environ.get("NVFP4_ABI_TEST_LIB")
    if alt:  # a separately built copy (the sanitizer run of tests/test_api_sanitizers.py)
        L = ctypes.CDLL(alt)
        for name, (args, res) in nvfp4.SIGNATURES.items():
            getattr(L, name).argtypes = args
            getattr(L, name).restype = res
        return L
    if not os.path.exists(nvfp4.LIB_PATH):
        build.build()
    return nvfp4.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"NVFP4_API\s+[^;(]*?\b((?:nvfp4|mxfp4)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["nvfp4_quantize", "nvfp4_dequantize", "nvfp4_quantize_kv_sink",
              "nvfp4_dequantize_kv_sink", "nvfp4_hadamard128", "nvfp4_workspace_bytes",
              "nvfp4_status_str", "nvfp4_abi_version", "nvfp4_global_scale",
              "nvfp4_kv_append", "nvfp4_quantize_rht", "mxfp4_quantize", "mxfp4_dequantize"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from microscaling_fp4_block_amd import nvfp4

    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in nvfp4.SIGNATURES, n


def test_version_and_status_text(lib):
    assert lib.nvfp4_abi_version() == 1
    texts = {lib.nvfp4_status_str(s).decode() for s in range(6)}
    assert len(texts) == 6
    assert lib.nvfp4_status_str(99).decode() == "unknown status"
    assert lib.nvfp4_workspace_bytes(8192, 28672, 0) >= 4 * 256
    assert lib.nvfp4_hw_self_check(None) == 1  # a null counts array: refused before any HIP call


P = 0x10000  # a well-aligned fake device address: every call below fails its checks first


def q(lib, **kw):
    a = dict(x=P, xdt=1, rows=4, cols=64, block=16, f_lo=-2, f_hi=6, flags=0, codes=P,
             scales=P, gs=P, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.nvfp4_quantize(a["x"], a["xdt"], a["rows"], a["cols"], a["block"], a["f_lo"],
                              a["f_hi"], a["flags"], a["codes"], a["scales"], a["gs"], a["ws"],
                              a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scales=None), 1), (dict(gs=None), 1),
    (dict(xdt=7), 1), (dict(block=32), 1), (dict(f_lo=1), 1), (dict(f_hi=-1), 1),
    (dict(f_lo=-127), 1), (dict(f_hi=127), 1), (dict(flags=8), 1),
    (dict(cols=24), 2), (dict(cols=0), 2), (dict(rows=-1), 2), (dict(rows=1 << 40), 2),
    (dict(flags=1, xdt=0), 1), (dict(flags=1, cols=64), 2),
    (dict(x=P + 8), 3), (dict(codes=P + 4), 3),
    (dict(ws=None), 4), (dict(wsb=16), 4),
])
def test_quantize_argument_checks(lib, kw, status):
    assert q(lib, **kw) == status


def q_noalloc(lib, **kw):
    a = dict(x=P, xdt=1, rows=4, cols=64, block=16, f_lo=-2, f_hi=6, flags=0, codes=P,
             scales=P, gs=P, stream=None)
    a.update(kw)
    return lib.nvfp4_quantize_noalloc(a["x"], a["xdt"], a["rows"], a["cols"], a["block"],
                                      a["f_lo"], a["f_hi"], a["flags"], a["codes"], a["scales"],
                                      a["gs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scales=None), 1), (dict(gs=None), 1),
    (dict(xdt=7), 1), (dict(block=32), 1), (dict(f_lo=1), 1), (dict(f_hi=-1), 1),
    (dict(f_lo=-127), 1), (dict(f_hi=127), 1), (dict(flags=8), 1),
    (dict(cols=24), 2), (dict(cols=0), 2), (dict(rows=-1), 2), (dict(rows=1 << 40), 2),
    (dict(flags=1, xdt=0), 1), (dict(flags=1, cols=64), 2),
    (dict(x=P + 8), 3), (dict(codes=P + 4), 3),
])
def test_quantize_noalloc_argument_checks(lib, kw, status):
    """The allocation-free quantize makes the same checks as nvfp4_quantize, before it
    looks up its device array."""
    assert q_noalloc(lib, **kw) == status
    assert lib.nvfp4_noalloc_scratch_bytes() == 2048


def test_dequantize_argument_checks(lib):
    f = lib.nvfp4_dequantize
    assert f(None, P, P, 4, 64, 16, P, 0, None) == 1
    assert f(P, P, P, 4, 64, 8, P, 0, None) == 1
    assert f(P, P, P, 4, 60, 16, P, 0, None) == 2
    assert f(P, P, P, 4, 64, 16, P + 4, 0, None) == 3
    assert f(P, P, P, 4, 64, 16, P, 5, None) == 1


def test_sink_argument_checks(lib):
    f = lib.nvfp4_quantize_kv_sink
    base = [P, 1, 1, 8, 300, 128, 128, 128, 16, -2, 6, 0, P, P, P, P, P, 1 << 20, None]
    a = list(base); a[6] = 200          # n_first + n_last > T
    assert f(*a) == 2
    a = list(base); a[5] = 120          # D not a multiple of 16
    assert f(*a) == 2
    a = list(base); a[15] = None        # sink missing
    assert f(*a) == 1
    g = lib.nvfp4_dequantize_kv_sink
    assert g(P, P, P, P, 1, 1, 8, 300, 128, 200, 128, 16, P, 0, None) == 2
    assert g(P, P, P, None, 1, 1, 8, 300, 128, 128, 128, 16, P, 0, None) == 1


def test_hadamard_argument_checks(lib):
    f = lib.nvfp4_hadamard128
    assert f(P, 0, 4, P, None) == 1     # FP32 input is not supported by the MFMA transform
    assert f(None, 1, 4, P, None) == 1
    assert f(P, 1, -1, P, None) == 2


def test_binding_refuses_cpu_tensors(lib):
    import torch

    import microscaling_fp4_block_amd as nv

    with pytest.raises(ValueError):
        nv.quantize(torch.zeros(4, 64))


def test_rht_argument_checks(lib):
    w = (ctypes.c_uint32 * 4)(1, 2, 3, 4)
    sp = ctypes.addressof(w)
    assert lib.nvfp4_hadamard128_rht(P, 1, 4, None, P, None) == 1   # signs required
    assert lib.nvfp4_hadamard128_rht(P, 0, 4, sp, P, None) == 1     # bf16 only
    assert lib.nvfp4_hadamard128_rht(P, 1, -1, sp, P, None) == 2
    q = lib.nvfp4_quantize_rht
    assert q(P, 1, 4, 256, 16, -2, 6, 0, None, P, P, P, P, 1 << 20, None) == 1
    assert q(P, 0, 4, 256, 16, -2, 6, 0, sp, P, P, P, P, 1 << 20, None) == 1   # FP32 input
    assert q(P, 1, 4, 192, 16, -2, 6, 0, sp, P, P, P, P, 1 << 20, None) == 2   # cols % 128
    assert lib.nvfp4_global_scale_rht(P, 1, 4, 256, 0, None, P, P, 1 << 20, None) == 1


def test_mxfp4_argument_checks(lib):
    q = lib.mxfp4_quantize
    assert q(P, 1, 4, 256, 16, 0, 0, P, P, None) == 1    # block must be 32
    assert q(P, 1, 4, 256, 32, -9, 0, P, P, None) == 1   # offsets within +-8
    assert q(P, 1, 4, 256, 32, 1, 2, P, P, None) == 1    # 0 inside the range
    assert q(P, 1, 4, 240, 32, 0, 0, P, P, None) == 2    # cols % 32
    assert q(P, 1, -1, 256, 32, 0, 0, P, P, None) == 2
    assert q(None, 1, 4, 256, 32, 0, 0, P, P, None) == 1
    assert q(P + 8, 1, 4, 256, 32, 0, 0, P, P, None) == 3
    assert q(P, 1, 0, 256, 32, 0, 0, None, None, None) == 0   # empty: nothing to do
    d = lib.mxfp4_dequantize
    assert d(P, P, 4, 256, 16, P, 0, None) == 1
    assert d(P, P, 4, 250, 32, P, 0, None) == 2
    assert d(P, P, 4, 256, 32, P + 4, 0, None) == 3


def test_attention_argument_checks(lib):
    f = lib.nvfp4_attention
    base = [P] * 9
    assert f(*base, 1, 2, 1, 64, 64, 64, 0, P, 0, None) == 2     # head dimension must be 128
    assert f(*base, 1, 3, 2, 64, 64, 128, 0, P, 0, None) == 2    # Hq % Hkv
    assert f(*base, 1, 2, 1, -1, 64, 128, 0, P, 0, None) == 2
    assert f(*base, 1, 2, 1, 64, 64, 128, 0, P, 7, None) == 1    # output dtype
    assert f(*([None] + [P] * 8), 1, 2, 1, 64, 64, 128, 0, P, 0, None) == 1
    assert f(*base, 1, 2, 1, 64, 64, 128, 0, P + 8, 0, None) == 3
    for i in (1, 4, 7):                                           # q, k, v scales: 8-byte words
        ptrs = list(base)
        ptrs[i] = P + 4
        assert f(*ptrs, 1, 2, 1, 64, 64, 128, 0, P, 0, None) == 3
    assert f(*base, 1, 2, 1, 0, 64, 128, 0, P, 0, None) == 0     # no queries: nothing to do


def test_attention_kv_cache_argument_checks(lib):
    f = lib.nvfp4_attention_kv_cache
    ptrs = [P] * 13
    # cache dtype must be bf16; head dimension 128; middle rows must fit cap
    assert f(*ptrs, 0, 1, 2, 1, 8, 300, 128, 16, 16, 64, P, 0, None) == 1
    assert f(*ptrs, 1, 1, 2, 1, 8, 300, 64, 16, 16, 300, P, 0, None) == 2
    assert f(*ptrs, 1, 1, 2, 1, 8, 300, 128, 16, 16, 100, P, 0, None) == 2
    assert f(*ptrs, 1, 1, 3, 2, 8, 300, 128, 16, 16, 300, P, 0, None) == 2
    assert f(*ptrs, 1, 1, 2, 1, 0, 300, 128, 16, 16, 300, P, 0, None) == 0
    for i in (1, 6, 11):                                          # q, k, v scales: 8-byte words
        bad = list(ptrs)
        bad[i] = P + 4
        assert f(*bad, 1, 1, 2, 1, 8, 300, 128, 16, 16, 300, P, 0, None) == 3


def test_largest_accepted_tensor(lib):
    """2^29 blocks of 16 (bf16 or FP32 [524288, 16384]) pass the shape checks: the
    call stops only at the too-small workspace, before any launch. One more row,
    or the same element count in rows of 16 (2^33 rows), is refused as a shape."""
    for xdt in (0, 1):
        assert q(lib, xdt=xdt, rows=524288, cols=16384, wsb=16) == 4
        assert q(lib, xdt=xdt, rows=524289, cols=16384, wsb=16) == 2
        assert q(lib, xdt=xdt, rows=1 << 29, cols=16, wsb=16) == 4
        assert q(lib, xdt=xdt, rows=(1 << 29) + 1, cols=16, wsb=16) == 2
    assert q(lib, rows=524288, cols=16384, wsb=16, flags=1) == 4  # Hadamard: same limit


def test_huge_dimensions_are_refused_without_overflow(lib):
    """Dimensions whose products or sums would overflow 64 bits are refused as shapes
    (the checks bound each factor before multiplying)."""
    big = 1 << 40
    q = lib.nvfp4_quantize_kv_sink
    assert q(P, 1, big, big, 8, 128, 0, 0, 16, -2, 6, 0, P, P, P, P, P, 1 << 20, None) == 2
    assert q(P, 1, 1, 1, 8, 128, 1 << 62, 1 << 62, 16, -2, 6, 0, P, P, P, P, P, 1 << 20, None) == 2
    d = lib.nvfp4_dequantize_kv_sink
    assert d(P, P, P, P, 1, big, big, 300, 128, 128, 128, 16, P, 0, None) == 2
    assert d(P, P, P, P, 1, 1, 1, 300, 128, 1 << 62, 1 << 62, 16, P, 0, None) == 2
    a = lib.nvfp4_kv_append
    assert a(P, 1, big, big, 8, 1, 128, 4, 4, 64, 16, -2, 6, 0, P, P, P, P, P, None) == 2
    assert a(P, 1, 1, 1, 1 << 62, 1 << 62, 128, 4, 4, 64, 16, -2, 6, 0, P, P, P, P, P, None) == 2
    assert a(P, 1, 1, 1, 8, 1, 128, 1 << 62, 4, 64, 16, -2, 6, 0, P, P, P, P, P, None) == 2
    f = lib.nvfp4_attention
    assert f(*([P] * 9), big, big, 1, 64, 64, 128, 0, P, 0, None) == 2
    c = lib.nvfp4_attention_kv_cache
    assert c(*([P] * 13), 1, big, big, 1, 8, 300, 128, 16, 16, 300, P, 0, None) == 2
    assert c(*([P] * 13), 1, 1, 2, 1, 8, 300, 128, 1 << 62, 1 << 62, 300, P, 0, None) == 2


def test_device_length_argument_checks(lib):
    a = lib.nvfp4_kv_append_dev
    base = [P, 1, 1, 2, 1, 128, 4, 4, 64, 16, -2, 6, 0, None, P, P, P, P, P, P, None]
    x = list(base); x[19] = None          # length missing
    assert a(*x) == 1
    x = list(base); x[19] = P + 4         # length not 8-byte aligned
    assert a(*x) == 3
    x = list(base); x[2] = 1 << 40; x[3] = 1 << 40
    assert a(*x) == 2
    x = list(base); x[4] = 0              # nothing to append: nothing enqueued
    assert a(*x) == 0
    c = lib.nvfp4_attention_kv_cache_dev
    assert c(*([P] * 13), 1, 1, 2, 1, 8, None, 128, 16, 16, 300, P, 0, None) == 1
    assert c(*([P] * 13), 1, 1, 2, 1, 8, P + 4, 128, 16, 16, 300, P, 0, None) == 3
    assert c(*([P] * 13), 1, 1, 2, 1, 0, P, 128, 16, 16, 300, P, 0, None) == 0


def test_split_attention_argument_checks(lib):
    w = lib.nvfp4_attention_split_workspace_bytes
    # (2 + ceil(cap / split)) units x B * Hq * Nq rows x 130 FP32 values
    assert w(1, 32, 1, 32768, 512) == (2 + 64) * 32 * 130 * 4
    assert w(2, 8, 3, 1000, 96) == (2 + 11) * 48 * 130 * 4
    assert w(1, 32, 1, 32768, 48) == 0          # split not a multiple of 32
    assert w(1, 32, 1, 32768, 0) == 0
    assert w(1, 32, 1, 1 << 30, 32) == 0        # more than 65535 units
    assert w(1, 1 << 40, 1, 100, 32) == 0
    need = w(1, 2, 8, 300, 64)
    for f, tokens in ((lib.nvfp4_attention_kv_cache_split, 300),
                      (lib.nvfp4_attention_kv_cache_split_dev, P)):
        args = lambda split, ws, nbytes, Nq=8: [*([P] * 13), 1, 1, 2, 1, Nq, tokens, 128, 16, 16,
                                                300, split, ws, nbytes, P, 0, None]
        assert f(*args(48, P, need)) == 1        # split must be a multiple of 32
        assert f(*args(0, P, need)) == 1         # and positive
        assert f(*args(64, None, need)) == 4     # workspace missing
        assert f(*args(64, P, need - 1)) == 4    # workspace too small
        assert f(*args(64, P + 4, need)) == 3    # workspace not 16-byte aligned
        assert f(*args(32, P, 1 << 40, Nq=0)) == 0   # no queries: nothing to do
    d = lib.nvfp4_attention_kv_cache_split_dev
    assert d(*([P] * 13), 1, 1, 2, 1, 8, None, 128, 16, 16, 300, 64, P, need, P, 0, None) == 1


def test_kv_append2_argument_checks(lib):
    """The paired K and V append checks both caches before it enqueues anything."""
    from microscaling_fp4_block_amd import nvfp4

    f = lib.nvfp4_kv_append2_dev
    ref = lambda length, scales=P: nvfp4._KvCacheRef(P, 0, None, P, P, P, P, scales, length)
    addr = ctypes.addressof
    shape = lambda t_new=1, D=128: [1, 1, 2, t_new, D, 16, 16, 64, 16, -2, 6, None]
    k, v = ref(P), ref(P + 64)
    assert f(None, addr(v), *shape()) == 1               # a cache missing
    same = ref(P)
    assert f(addr(k), addr(same), *shape()) == 1         # one length word for both
    assert f(addr(k), addr(v), *shape(D=100)) == 2       # D % 16
    bad = ref(P + 68)
    assert f(addr(k), addr(bad), *shape()) == 3          # V's length not 8-byte aligned
    assert f(addr(k), addr(v), *shape(t_new=0)) == 0     # nothing to append: no launch


def _call(fn, names, defaults, kw):
    a = {**defaults, **kw}
    return fn(*[a[n] for n in names])


def test_balance_argument_checks(lib):
    """The balancing pair's entry points check on the host before any launch."""
    qn = ("x", "xdt", "rows", "cols", "block", "f_lo", "f_hi", "flags", "e", "signs", "codes",
          "scales", "gs", "ws", "wsb", "stream")
    qd = dict(x=P, xdt=1, rows=4, cols=128, block=16, f_lo=-2, f_hi=6, flags=0, e=P, signs=None,
              codes=P, scales=P, gs=P, ws=P, wsb=1 << 20, stream=None)
    bq = lambda **kw: _call(lib.nvfp4_quantize_balanced, qn, qd, kw)
    assert bq(e=None) == 1                      # no exponents
    assert bq(flags=8) == 1                     # unknown flag
    assert bq(signs=P) == 1                     # signs without the transform
    assert bq(flags=1, cols=256) == 2           # transform needs cols == 128
    assert bq(flags=1, xdt=0) == 1              # transform needs bf16
    assert bq(e=P + 8) == 3                     # exponents 16-byte aligned
    assert bq(wsb=16) == 4
    assert bq(cols=24) == 2
    ws = lib.nvfp4_balance_workspace_bytes
    assert ws(128) == 2 * 256 * 128 * 8 and ws(0) == 0 and ws(4096) == 0
    en = ("q", "k", "dt", "rq", "rk", "cols", "e", "ws", "wsb", "stream")
    ed = dict(q=P, k=P, dt=1, rq=8, rk=8, cols=128, e=P, ws=P, wsb=1 << 20, stream=None)
    be = lambda **kw: _call(lib.nvfp4_balance_exponents, en, ed, kw)
    assert be(e=None) == 1 and be(dt=5) == 1 and be(q=None) == 1
    assert be(cols=24) == 2 and be(cols=4096) == 2 and be(rq=-1) == 2
    assert be(k=P + 4) == 3
    assert be(wsb=1024) == 4 and be(ws=P + 4) == 4
    hn = ("x", "xdt", "rows", "e", "flags", "signs", "y", "stream")
    hd = dict(x=P, xdt=1, rows=4, e=P, flags=0, signs=None, y=P, stream=None)
    hb = lambda **kw: _call(lib.nvfp4_hadamard128_balanced, hn, hd, kw)
    assert hb(xdt=0) == 1 and hb(e=None) == 1 and hb(flags=1) == 1 and hb(rows=-1) == 2
    assert hb(y=P + 4) == 3
