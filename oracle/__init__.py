"""CPU oracle for the packed trellis-coded linear layer (ctypes wrapper).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code
with the GPU library (trellis_coded_quantized_amd) and never imports it.

Every function forwards to trellis_oracle.c, whose comments cite the
defining passage of the pages for each step.  Arrays are numpy; bf16 and
fp16 values travel as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u32p = ctypes.POINTER(ctypes.c_uint32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i16p = ctypes.POINTER(ctypes.c_int16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "tro_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "tro_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "tro_double_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
        "tro_state": (ctypes.c_uint32, [_u32p, _int, _int, _int, _int]),
        "tro_y": (ctypes.c_int32, [ctypes.c_uint32]),
        "tro_value": (ctypes.c_float, [ctypes.c_int32]),
        "tro_decode": (None, [_u32p, _i64, _i64, _int, _int, _int, _u16p, _i16p, _f32p]),
        "tro_matvec_axis1": (None, [_u32p, _u16p, _u16p, _int, _i64, _i64, _int, _int, _int,
                                    _i64p, _i64, _f64p, _f64p]),
        "tro_matvec_axis0": (None, [_u32p, _u16p, _u16p, _int, _i64, _i64, _int, _int, _int,
                                    _i64p, _i64, _f64p, _f64p]),
        "tro_swiglu": (ctypes.c_uint16, [ctypes.c_double, ctypes.c_double]),
        "tro_gateup_swiglu": (None, [_u32p, _u16p, _u32p, _u16p, _u16p, _int, _i64, _i64, _int,
                                     _int, _int, _i64p, _i64, _f64p, _f64p, _u16p, _f64p, _f64p]),
        "tro_expand_bf16": (None, [_u32p, _u16p, _i64, _i64, _int, _int, _int, _i64, _i64, _u16p]),
        "tro_prefill": (None, [_u32p, _u16p, _u16p, _i64, _i64, _i64, _int, _int, _int,
                               _i64p, _i64, _i64p, _i64, _f64p, _f64p]),
        "tro_prefill_axis0": (None, [_u32p, _u16p, _u16p, _i64, _i64, _i64, _int, _int, _int,
                                     _i64p, _i64, _i64p, _i64, _f64p, _f64p]),
        "tro_num_threads": (_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctype) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return _load().tro_num_threads()


# ---- scalar conversions -------------------------------------------------

def half_to_double(h: int) -> float:
    return _load().tro_half_to_double(int(h))


def bf16_to_double(b: int) -> float:
    return _load().tro_bf16_to_double(int(b))


def double_to_bf16(v: float) -> int:
    return int(_load().tro_double_to_bf16(float(v)))


def bf16_round_array(v: np.ndarray) -> np.ndarray:
    """Elementwise round-to-nearest-even bf16 bits of a float64 array."""
    lib = _load()
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.fromiter((lib.tro_double_to_bf16(float(t)) for t in flat), dtype=np.uint16,
                      count=flat.size)
    return out.reshape(np.shape(v))


# ---- decode primitive ---------------------------------------------------

def state(block: np.ndarray, k: int, L: int, T: int, t: int) -> int:
    b = _c(block, np.uint32)
    return int(_load().tro_state(_ptr(b, _u32p), k, L, T, t))


def code_y(s: int) -> int:
    return int(_load().tro_y(int(s)))


def code_value(y: int) -> np.float32:
    return np.float32(_load().tro_value(int(y)))


def decode(codes: np.ndarray, R: int, C: int, k: int, L: int, T: int):
    """(states uint16 [R, C], y int16 [R, C], values float32 [R, C])."""
    c = _c(codes, np.uint32)
    st = np.empty((R, C), np.uint16)
    ys = np.empty((R, C), np.int16)
    vals = np.empty((R, C), np.float32)
    _load().tro_decode(_ptr(c, _u32p), R, C, k, L, T, _ptr(st, _u16p), _ptr(ys, _i16p),
                       _ptr(vals, _f32p))
    return st, ys, vals


# ---- layer results ------------------------------------------------------

def _sel(sel, n):
    if sel is None:
        return None, n
    s = _c(sel, np.int64)
    return s, s.size


def _abs_buf(shape, with_abs):
    return np.empty(shape, np.float64) if with_abs else None


def matvec_axis1(codes, scales, x, M, R, C, k, L, T, rows=None, with_abs=False):
    """float64 [M, nrows] exact-in-double sums (axis 1, coded along inputs);
    with_abs: (sums, sums of |term|)."""
    c, s, xx = _c(codes, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    sel, n = _sel(rows, R)
    out = np.empty((M, n), np.float64)
    ab = _abs_buf((M, n), with_abs)
    _load().tro_matvec_axis1(_ptr(c, _u32p), _ptr(s, _u16p), _ptr(xx, _u16p), M, R, C, k, L, T,
                             _ptr(sel, _i64p), n, _ptr(out, _f64p), _ptr(ab, _f64p))
    return (out, ab) if with_abs else out


def matvec_axis0(codes, scales, x, M, R, C, k, L, T, cols=None, with_abs=False):
    """float64 [M, ncols] sums for the axis-0 (stored transpose) layout;
    with_abs: (sums, sums of |term|)."""
    c, s, xx = _c(codes, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    sel, n = _sel(cols, C)
    out = np.empty((M, n), np.float64)
    ab = _abs_buf((M, n), with_abs)
    _load().tro_matvec_axis0(_ptr(c, _u32p), _ptr(s, _u16p), _ptr(xx, _u16p), M, R, C, k, L, T,
                             _ptr(sel, _i64p), n, _ptr(out, _f64p), _ptr(ab, _f64p))
    return (out, ab) if with_abs else out


def swiglu(gate: float, up: float) -> int:
    return int(_load().tro_swiglu(float(gate), float(up)))


def gateup_swiglu(gcodes, gscales, ucodes, uscales, x, M, R, C, k, L, T, rows=None, with_abs=False):
    """(gate float64 [M, n], up float64 [M, n], out bf16 bits [M, n]); with_abs
    appends the gate's and the up projection's sums of |term|."""
    gc, gs = _c(gcodes, np.uint32), _c(gscales, np.uint16)
    uc, us = _c(ucodes, np.uint32), _c(uscales, np.uint16)
    xx = _c(x, np.uint16)
    sel, n = _sel(rows, R)
    g = np.empty((M, n), np.float64)
    u = np.empty((M, n), np.float64)
    o = np.empty((M, n), np.uint16)
    ga, ua = _abs_buf((M, n), with_abs), _abs_buf((M, n), with_abs)
    _load().tro_gateup_swiglu(_ptr(gc, _u32p), _ptr(gs, _u16p), _ptr(uc, _u32p), _ptr(us, _u16p),
                              _ptr(xx, _u16p), M, R, C, k, L, T, _ptr(sel, _i64p), n,
                              _ptr(g, _f64p), _ptr(u, _f64p), _ptr(o, _u16p), _ptr(ga, _f64p), _ptr(ua, _f64p))
    return (g, u, o, ga, ua) if with_abs else (g, u, o)


def expand_bf16(codes, scales, R, C, k, L, T, r0=0, nr=None) -> np.ndarray:
    """bf16 bits [nr, C] of stored rows r0 .. r0+nr-1."""
    if nr is None:
        nr = R - r0
    c, s = _c(codes, np.uint32), _c(scales, np.uint16)
    out = np.empty((nr, C), np.uint16)
    _load().tro_expand_bf16(_ptr(c, _u32p), _ptr(s, _u16p), R, C, k, L, T, r0, nr,
                            _ptr(out, _u16p))
    return out


def prefill_sums(codes, scales, x, M, R, C, k, L, T, ms, rows, with_abs=False):
    """float64 [len(ms), len(rows)] sums of bf16 weights times bf16 x;
    with_abs: (sums, sums of |term|)."""
    c, s, xx = _c(codes, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    msa, rsa = _c(ms, np.int64), _c(rows, np.int64)
    out = np.empty((msa.size, rsa.size), np.float64)
    ab = _abs_buf(out.shape, with_abs)
    _load().tro_prefill(_ptr(c, _u32p), _ptr(s, _u16p), _ptr(xx, _u16p), M, R, C, k, L, T,
                        _ptr(msa, _i64p), msa.size, _ptr(rsa, _i64p), rsa.size, _ptr(out, _f64p),
                        _ptr(ab, _f64p))
    return (out, ab) if with_abs else out


def prefill_axis0_sums(codes, scales, x, M, R, C, k, L, T, ms, cols, with_abs=False):
    """float64 [len(ms), len(cols)] sums over the stored rows of bf16 weights
    times bf16 x, for a matrix stored transposed (axis 0); with_abs: (sums,
    sums of |term|)."""
    c, s, xx = _c(codes, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    msa, csa = _c(ms, np.int64), _c(cols, np.int64)
    out = np.empty((msa.size, csa.size), np.float64)
    ab = _abs_buf(out.shape, with_abs)
    _load().tro_prefill_axis0(_ptr(c, _u32p), _ptr(s, _u16p), _ptr(xx, _u16p), M, R, C, k, L, T,
                              _ptr(msa, _i64p), msa.size, _ptr(csa, _i64p), csa.size, _ptr(out, _f64p),
                              _ptr(ab, _f64p))
    return (out, ab) if with_abs else out
