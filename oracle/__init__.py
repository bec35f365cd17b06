"""CPU oracle for the 2-bit PhaseQuant complex linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package; the product path never
does.  Thin numpy wrappers around oracle/liboracle.so (plain C, double
precision, exact integers); see fairy_oracle.h for what each call computes
and which passage of the pages it follows.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ROW16 = 0
TILED64 = 1

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_version.restype = _i32
        L.orc_set_threads.argtypes = [_i32]
        L.orc_set_threads.restype = _i32
        L.orc_phase_code.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_phase_code.restype = _i32
        L.orc_real_to_complex.argtypes = [_p, _i64, _i64, _p, _p, _p, _p]
        L.orc_real_to_complex_f32.argtypes = [_p, _i64, _i64, _p, _p, _p, _p]
        L.orc_abs_mean.argtypes = [_p, _p, _i64]
        L.orc_abs_mean.restype = ctypes.c_float
        L.orc_phasequant.argtypes = [_p, _p, _i64, _i32, _p, _p, _p, _p]
        L.orc_packed_words.argtypes = [_i64, _i64, _i32, _i32]
        L.orc_packed_words.restype = _i64
        L.orc_pack.argtypes = [_p, _i32, _i64, _i64, _i32, _p]
        L.orc_unpack.argtypes = [_p, _i32, _i64, _i64, _i32, _p]
        L.orc_cgemv_dense.argtypes = [_p, _p, _i32, _i32, _i64, _i64, _p, _p, _i32, _i64, _p, _p, _i64]
        L.orc_cgemv_acc.argtypes = [_p, _p, _i32, _i32, _i64, _i64, _p, _p, _i32, _i64, _p, _p, _p, _i64]
        L.orc_cgemv_acc_i64.argtypes = [_p, _i32, _i64, _i64, _p, _p, _i32, _i64, _p]
        L.orc_cattn_scores.argtypes = [_p, _p, _p, _p, _i32, _i64, _i64, _i32, ctypes.c_double, _i32, _p]
        L.orc_cattention.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i64, _i64, _i32, ctypes.c_double, _i32,
                                     _p, _p]
        L.orc_rope.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i32, ctypes.c_double]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def set_threads(n: int) -> int:
    return lib().orc_set_threads(int(n))


def phase_code(re: float, im: float) -> int:
    return lib().orc_phase_code(float(re), float(im))


def phase_codes(w_re, w_im):
    """Vector form of phase_code (loops in C through orc_phasequant is not
    used here: codes of a single stage are the stage-1 codes)."""
    w_re = np.ascontiguousarray(w_re, np.float32).ravel()
    w_im = np.ascontiguousarray(w_im, np.float32).ravel()
    codes = np.empty(w_re.size, np.uint8)
    scales = np.empty(2, np.float32)
    lib().orc_phasequant(w_re.ctypes.data, w_im.ctypes.data, w_re.size, 1,
                         codes.ctypes.data, scales.ctypes.data, None, None)
    return codes


def real_to_complex(R, n: int, m: int, f32: bool = False):
    R, pR = _c(R, np.float32)
    assert R.size == 4 * n * m
    dt = np.float32 if f32 else np.float64
    outs = [np.empty((n, m), dt) for _ in range(4)]
    fn = lib().orc_real_to_complex_f32 if f32 else lib().orc_real_to_complex
    fn(pR, n, m, *[o.ctypes.data for o in outs])
    return tuple(outs)  # u_re, u_im, w_re, w_im


def abs_mean(v, sel) -> np.float32:
    v, pv = _c(v, np.float32)
    s, ps = _c(sel, np.uint8)
    assert v.size == s.size
    return np.float32(lib().orc_abs_mean(pv, ps, v.size))


def phasequant(w_re, w_im, stages: int, want_resid: bool = True):
    w_re, pr = _c(w_re, np.float32)
    w_im, pi = _c(w_im, np.float32)
    shape = w_re.shape
    cnt = w_re.size
    codes = np.empty((stages,) + shape, np.uint8)
    scales = np.empty((stages, 2), np.float32)
    rr = np.empty(shape, np.float32) if want_resid else None
    ri = np.empty(shape, np.float32) if want_resid else None
    lib().orc_phasequant(pr, pi, cnt, stages, codes.ctypes.data, scales.ctypes.data,
                         rr.ctypes.data if want_resid else None,
                         ri.ctypes.data if want_resid else None)
    return codes, scales, rr, ri


def packed_words(rows: int, m: int, planes: int, layout: int) -> int:
    return lib().orc_packed_words(rows, m, planes, layout)


def pack(codes, layout: int):
    """codes: uint8 [planes][rows][m] -> uint32 words of the layout."""
    codes, pc = _c(codes, np.uint8)
    planes, rows, m = codes.shape
    out = np.empty(packed_words(rows, m, planes, layout), np.uint32)
    lib().orc_pack(pc, planes, rows, m, layout, out.ctypes.data)
    return out


def unpack(packed, planes: int, rows: int, m: int, layout: int):
    packed, pp = _c(packed, np.uint32)
    out = np.empty((planes, rows, m), np.uint8)
    lib().orc_unpack(pp, planes, rows, m, layout, out.ctypes.data)
    return out


def cgemv_dense(codes, scales, stages: int, has_conj: bool, x_re, x_im):
    """codes [P][n][m], scales [P][2], x [B][m] (any real dtype, converted
    exactly to double) -> y_re, y_im [B][n] (float64)."""
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.float32)
    P, n, m = codes.shape
    assert P == stages * (2 if has_conj else 1)
    x_re, pxr = _c(np.atleast_2d(x_re), np.float64)
    x_im, pxi = _c(np.atleast_2d(x_im), np.float64)
    B = x_re.shape[0]
    assert x_re.shape == (B, m) and x_im.shape == (B, m)
    y_re = np.empty((B, n)); y_im = np.empty((B, n))
    lib().orc_cgemv_dense(pc, ps, stages, int(has_conj), n, m, pxr, pxi, B, m,
                          y_re.ctypes.data, y_im.ctypes.data, n)
    return y_re, y_im


def cgemv_acc(codes, scales, stages: int, has_conj: bool, x_re, x_im):
    """Four-accumulator form.  Returns (acc [P][4][B][n], y_re, y_im)."""
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.float32)
    P, n, m = codes.shape
    x_re, pxr = _c(np.atleast_2d(x_re), np.float64)
    x_im, pxi = _c(np.atleast_2d(x_im), np.float64)
    B = x_re.shape[0]
    acc = np.empty((P, 4, B, n))
    y_re = np.empty((B, n)); y_im = np.empty((B, n))
    lib().orc_cgemv_acc(pc, ps, stages, int(has_conj), n, m, pxr, pxi, B, m,
                        acc.ctypes.data, y_re.ctypes.data, y_im.ctypes.data, n)
    return acc, y_re, y_im


def cgemv_acc_i64(codes, x_re, x_im):
    """int8 activations -> exact int64 accumulators [P][4][B][n]."""
    codes, pc = _c(codes, np.uint8)
    P, n, m = codes.shape
    x_re, pxr = _c(np.atleast_2d(x_re), np.int8)
    x_im, pxi = _c(np.atleast_2d(x_im), np.int8)
    B = x_re.shape[0]
    acc = np.empty((P, 4, B, n), np.int64)
    lib().orc_cgemv_acc_i64(pc, P, n, m, pxr, pxi, B, m, acc.ctypes.data)
    return acc


def _attn_args(q_re, q_im, k_re, k_im):
    q_re, pqr = _c(q_re, np.float32)
    q_im, pqi = _c(q_im, np.float32)
    k_re, pkr = _c(k_re, np.float32)
    k_im, pki = _c(k_im, np.float32)
    heads, sq, d = q_re.shape
    sk = k_re.shape[1]
    assert q_im.shape == q_re.shape and k_re.shape == (heads, sk, d) and k_im.shape == k_re.shape
    return (q_re, q_im, k_re, k_im), (pqr, pqi, pkr, pki), heads, sq, sk, d


def cattn_scores(q_re, q_im, k_re, k_im, scale: float, causal: bool = False):
    """[heads][sq][d] queries, [heads][sk][d] keys -> scores [heads][sq][sk] (float64)."""
    keep, ptrs, heads, sq, sk, d = _attn_args(q_re, q_im, k_re, k_im)
    s = np.empty((heads, sq, sk), np.float64)
    lib().orc_cattn_scores(*ptrs, heads, sq, sk, d, float(scale), int(bool(causal)), s.ctypes.data)
    return s


def cattention(q_re, q_im, k_re, k_im, v_re, v_im, scale: float, causal: bool = False):
    """Complex attention forward -> (o_re, o_im) [heads][sq][d] (float64)."""
    keep, ptrs, heads, sq, sk, d = _attn_args(q_re, q_im, k_re, k_im)
    v_re, pvr = _c(v_re, np.float32)
    v_im, pvi = _c(v_im, np.float32)
    assert v_re.shape == (heads, sk, d) and v_im.shape == v_re.shape
    o_re = np.empty((heads, sq, d), np.float64)
    o_im = np.empty((heads, sq, d), np.float64)
    lib().orc_cattention(*ptrs, pvr, pvi, heads, sq, sk, d, float(scale), int(bool(causal)), o_re.ctypes.data,
                         o_im.ctypes.data)
    return o_re, o_im


def rope(y_re, y_im, positions, head_dim: int, base: float):
    """y [rows][n] complex (two float arrays) -> rotated copies (float64)."""
    y_re = np.array(np.atleast_2d(y_re), np.float64, order="C")
    y_im = np.array(np.atleast_2d(y_im), np.float64, order="C")
    pos, pp = _c(positions, np.int32)
    rows, n = y_re.shape
    assert pos.size == rows and y_im.shape == y_re.shape
    lib().orc_rope(y_re.ctypes.data, y_im.ctypes.data, rows, n, n, pp, int(head_dim), float(base))
    return y_re, y_im
