"""ctypes binding of libfairy (include/fairy.h): argument marshalling only.

Every function has the C entry point's name and argument order.  Device
buffers may be given as torch tensors (their data_ptr() is passed) or as raw
integer addresses; `stream` is a torch.cuda.Stream, a raw hipStream_t integer
or None (torch's current stream when torch is loaded, else the null stream).
A non-OK status raises FairyError.  There is no fallback: if libfairy.so is
missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfairy.so")

FAIRY_OK = 0
FAIRY_ERR_INVALID_ARG = 1
FAIRY_ERR_UNSUPPORTED = 2
FAIRY_ERR_HIP = 3
FAIRY_ERR_WORKSPACE = 4

FAIRY_LAYOUT_ROW16 = 0
FAIRY_LAYOUT_TILED64 = 1

FAIRY_F32 = 0
FAIRY_BF16 = 1
FAIRY_I8 = 2

FAIRY_ALGO_AUTO = 0
FAIRY_ALGO_VALU = 1
FAIRY_ALGO_MFMA = 2


class FairyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class fairy_clinear(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64), ("m", ctypes.c_int64),
        ("stages", ctypes.c_int32), ("has_conj", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
    ]


class fairy_layer_info(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64), ("m", ctypes.c_int64),
        ("stages", ctypes.c_int32), ("has_conj", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("planes", ctypes.c_int32),
        ("packed_bytes", ctypes.c_uint64), ("header_bytes", ctypes.c_uint32),
    ]


_lib = None
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_complex_weight_amd.build`")
        # PyTorch ships its own HIP runtime (libamdhip64.so.7).  Load it first so
        # that libfairy binds to the same runtime instance that owns the device
        # memory and streams it is given; two runtimes in one process do not
        # share contexts.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        L.fairy_abi_version.restype = _i32
        L.fairy_status_string.argtypes = [_i32]
        L.fairy_status_string.restype = ctypes.c_char_p
        L.fairy_real_to_complex.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _p]
        L.fairy_real_to_complex.restype = _i32
        L.fairy_phasequant_workspace_bytes.argtypes = [_i64, _i32]
        L.fairy_phasequant_workspace_bytes.restype = _sz
        L.fairy_phasequant.argtypes = [_p, _p, _i64, _i32, _p, _p, _p, _p, _p, _sz, _p]
        L.fairy_phasequant.restype = _i32
        L.fairy_phasequant_noalloc.argtypes = [_p, _p, _i64, _i32, _p, _p, _p, _p, _p]
        L.fairy_phasequant_noalloc.restype = _i32
        L.fairy_packed_words.argtypes = [_i64, _i64, _i32, _i32]
        L.fairy_packed_words.restype = _i64
        L.fairy_pack.argtypes = [_p, _i32, _i64, _i64, _i32, _p, _p]
        L.fairy_pack.restype = _i32
        L.fairy_unpack.argtypes = [_p, _i32, _i64, _i64, _i32, _p, _p]
        L.fairy_unpack.restype = _i32
        L.fairy_cgemv_workspace_bytes.argtypes = [ctypes.POINTER(fairy_clinear), _i32, _i32]
        L.fairy_cgemv_workspace_bytes.restype = _sz
        L.fairy_cgemv.argtypes = [ctypes.POINTER(fairy_clinear), _p, _p, _i32, _i32, _i64, _p, _p, _i64, _p,
                                  _p, _sz, _p]
        L.fairy_cgemv.restype = _i32
        L.fairy_cgemv_group.argtypes = [ctypes.POINTER(fairy_clinear), _i32, _p, _p, _i32, _i32, _i64, _p, _p, _p, _p]
        L.fairy_cgemv_group.restype = _i32
        L.fairy_cgemm_workspace_bytes.argtypes = [ctypes.POINTER(fairy_clinear), _i64, _i32, _i32]
        L.fairy_cgemm_workspace_bytes.restype = _sz
        L.fairy_cgemm.argtypes = [ctypes.POINTER(fairy_clinear), _p, _p, _i32, _i64, _i64, _p, _p, _i64, _p,
                                  _i32, _p, _sz, _p]
        L.fairy_cgemm.restype = _i32
        L.fairy_quantize_workspace_bytes.argtypes = [_i64, _i64, _i32, _i32]
        L.fairy_quantize_workspace_bytes.restype = _sz
        L.fairy_quantize_real.argtypes = [_p, _i64, _i64, _i32, _p, _p, _p, _sz, _p]
        L.fairy_quantize_real.restype = _i32
        L.fairy_quantize_complex.argtypes = [_p, _p, _i64, _i64, _i32, _p, _p, _p, _sz, _p]
        L.fairy_quantize_complex.restype = _i32
        L.fairy_layer_file_bytes.argtypes = [_i64, _i64, _i32, _i32]
        L.fairy_layer_file_bytes.restype = _sz
        L.fairy_layer_save.argtypes = [ctypes.POINTER(fairy_clinear), _p, _sz, _p]
        L.fairy_layer_save.restype = _i32
        L.fairy_layer_read_info.argtypes = [_p, _sz, ctypes.POINTER(fairy_layer_info)]
        L.fairy_layer_read_info.restype = _i32
        L.fairy_layer_load.argtypes = [_p, _sz, _p, _p, _p]
        L.fairy_layer_load.restype = _i32
        L.fairy_cattention.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i64, _i64, _i32, ctypes.c_float, _i32,
                                       _p, _p, _p]
        L.fairy_cattention.restype = _i32
        L.fairy_cgemv_rope.argtypes = [ctypes.POINTER(fairy_clinear), _p, _p, _i32, _i32, _i64, _p, _p, _i64, _p, _i32,
                                       ctypes.c_float, _p]
        L.fairy_cgemv_rope.restype = _i32
        L.fairy_cgemm_rope.argtypes = [ctypes.POINTER(fairy_clinear), _p, _p, _i32, _i64, _i64, _p, _p, _i64, _i32, _p,
                                       _i32, ctypes.c_float, _p]
        L.fairy_cgemm_rope.restype = _i32
        L.fairy_cgemv_lut_workspace_bytes.argtypes = [ctypes.POINTER(fairy_clinear)]
        L.fairy_cgemv_lut_workspace_bytes.restype = _sz
        L.fairy_cgemv_lut.argtypes = [ctypes.POINTER(fairy_clinear), _p, _p, _i32, _p, _p, _p, _sz, _p]
        L.fairy_cgemv_lut.restype = _i32
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is not None:
        if getattr(x, "is_cuda", True) is False:
            raise ValueError("libfairy takes device buffers; got a host tensor")
        return dp()
    raise TypeError(f"expected a device tensor or an integer address, got {type(x).__name__}")


def _stream(s):
    if s is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str):
    if status != FAIRY_OK:
        raise FairyError(status, where)


def status_string(status: int) -> str:
    return lib().fairy_status_string(int(status)).decode()


def fairy_abi_version() -> int:
    return lib().fairy_abi_version()


def fairy_status_string(status: int) -> str:
    return status_string(status)


def fairy_real_to_complex(R, n, m, u_re, u_im, w_re, w_im, stream=None):
    _check(lib().fairy_real_to_complex(_ptr(R), n, m, _ptr(u_re), _ptr(u_im), _ptr(w_re), _ptr(w_im),
                                       _stream(stream)), "fairy_real_to_complex")


def fairy_phasequant_workspace_bytes(count, stages) -> int:
    return lib().fairy_phasequant_workspace_bytes(count, stages)


def fairy_phasequant(w_re, w_im, count, stages, codes, scales, resid_re, resid_im, workspace, workspace_bytes,
                     stream=None):
    _check(lib().fairy_phasequant(_ptr(w_re), _ptr(w_im), count, stages, _ptr(codes), _ptr(scales),
                                  _ptr(resid_re), _ptr(resid_im), _ptr(workspace), workspace_bytes,
                                  _stream(stream)), "fairy_phasequant")


def fairy_phasequant_noalloc(w_re, w_im, count, stages, codes, scales, resid_re=None, resid_im=None, stream=None):
    _check(lib().fairy_phasequant_noalloc(_ptr(w_re), _ptr(w_im), count, stages, _ptr(codes), _ptr(scales),
                                          _ptr(resid_re), _ptr(resid_im), _stream(stream)),
           "fairy_phasequant_noalloc")


def fairy_packed_words(rows, m, planes, layout) -> int:
    return lib().fairy_packed_words(rows, m, planes, layout)


def fairy_pack(codes, planes, rows, m, layout, packed, stream=None):
    _check(lib().fairy_pack(_ptr(codes), planes, rows, m, layout, _ptr(packed), _stream(stream)), "fairy_pack")


def fairy_unpack(packed, planes, rows, m, layout, codes, stream=None):
    _check(lib().fairy_unpack(_ptr(packed), planes, rows, m, layout, _ptr(codes), _stream(stream)),
           "fairy_unpack")


def make_clinear(n, m, stages, has_conj, packed, scales, layout=FAIRY_LAYOUT_TILED64) -> fairy_clinear:
    """Descriptor of a quantised layer; the caller keeps the buffers alive."""
    return fairy_clinear(int(n), int(m), int(stages), int(has_conj), int(layout), _ptr(packed), _ptr(scales))


def fairy_cgemv_workspace_bytes(L, batch, xdtype) -> int:
    return lib().fairy_cgemv_workspace_bytes(ctypes.byref(L), batch, xdtype)


def fairy_cgemv(L, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, acc=None, workspace=None,
                workspace_bytes=0, stream=None):
    _check(lib().fairy_cgemv(ctypes.byref(L), _ptr(x_re), _ptr(x_im), xdtype, batch, ldx, _ptr(y_re), _ptr(y_im),
                             ldy, _ptr(acc), _ptr(workspace), workspace_bytes, _stream(stream)), "fairy_cgemv")


def fairy_cgemv_group(layers, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, stream=None):
    """layers, y_re, y_im, ldy: sequences of the same length (descriptors,
    device buffers, leading dimensions)."""
    k = len(layers)
    if not (len(y_re) == len(y_im) == len(ldy) == k):
        raise ValueError("fairy_cgemv_group: layers, y_re, y_im and ldy differ in length")
    arr = (fairy_clinear * k)(*layers)
    yr = (_p * k)(*[_ptr(v) for v in y_re])
    yi = (_p * k)(*[_ptr(v) for v in y_im])
    ld = (_i64 * k)(*[int(v) for v in ldy])
    _check(lib().fairy_cgemv_group(arr, k, _ptr(x_re), _ptr(x_im), xdtype, batch, ldx, ctypes.cast(yr, _p),
                                   ctypes.cast(yi, _p), ctypes.cast(ld, _p), _stream(stream)), "fairy_cgemv_group")


def fairy_cgemm_workspace_bytes(L, M, xdtype, algo) -> int:
    return lib().fairy_cgemm_workspace_bytes(ctypes.byref(L), M, xdtype, algo)


def fairy_cgemm(L, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, acc=None, algo=FAIRY_ALGO_AUTO, workspace=None,
                workspace_bytes=0, stream=None):
    _check(lib().fairy_cgemm(ctypes.byref(L), _ptr(x_re), _ptr(x_im), xdtype, M, ldx, _ptr(y_re), _ptr(y_im), ldy,
                             _ptr(acc), algo, _ptr(workspace), workspace_bytes, _stream(stream)), "fairy_cgemm")


def fairy_quantize_workspace_bytes(n, m, stages, has_conj) -> int:
    return lib().fairy_quantize_workspace_bytes(n, m, stages, has_conj)


def fairy_quantize_real(R, n, m, stages, packed, scales, workspace, workspace_bytes, stream=None):
    _check(lib().fairy_quantize_real(_ptr(R), n, m, stages, _ptr(packed), _ptr(scales), _ptr(workspace),
                                     workspace_bytes, _stream(stream)), "fairy_quantize_real")


def fairy_quantize_complex(w_re, w_im, n, m, stages, packed, scales, workspace, workspace_bytes, stream=None):
    _check(lib().fairy_quantize_complex(_ptr(w_re), _ptr(w_im), n, m, stages, _ptr(packed), _ptr(scales),
                                        _ptr(workspace), workspace_bytes, _stream(stream)), "fairy_quantize_complex")


def fairy_layer_file_bytes(n, m, stages, has_conj) -> int:
    return lib().fairy_layer_file_bytes(n, m, stages, has_conj)


def _host_buf(buf):
    """A writable or readable host buffer (bytearray, bytes, numpy array) ->
    (address, size); the caller keeps it alive."""
    if isinstance(buf, (bytes, bytearray)):
        c = (ctypes.c_char * len(buf)).from_buffer(buf) if isinstance(buf, bytearray) else ctypes.c_char_p(buf)
        return ctypes.cast(c, ctypes.c_void_p).value, len(buf)
    iface = getattr(buf, "__array_interface__", None)
    if iface is not None:
        return iface["data"][0], buf.nbytes
    raise TypeError(f"expected bytes, bytearray or a numpy array, got {type(buf).__name__}")


def fairy_layer_save(L, buf, stream=None):
    addr, size = _host_buf(buf)
    _check(lib().fairy_layer_save(ctypes.byref(L), addr, size, _stream(stream)), "fairy_layer_save")


def fairy_layer_read_info(buf) -> fairy_layer_info:
    addr, size = _host_buf(buf)
    info = fairy_layer_info()
    _check(lib().fairy_layer_read_info(addr, size, ctypes.byref(info)), "fairy_layer_read_info")
    return info


def fairy_layer_load(buf, packed, scales, stream=None):
    addr, size = _host_buf(buf)
    _check(lib().fairy_layer_load(addr, size, _ptr(packed), _ptr(scales), _stream(stream)), "fairy_layer_load")


def fairy_cattention(q_re, q_im, k_re, k_im, v_re, v_im, dtype, heads, sq, sk, d, scale, causal, o_re, o_im,
                     stream=None):
    _check(lib().fairy_cattention(_ptr(q_re), _ptr(q_im), _ptr(k_re), _ptr(k_im), _ptr(v_re), _ptr(v_im), dtype,
                                  heads, sq, sk, d, float(scale), int(causal), _ptr(o_re), _ptr(o_im),
                                  _stream(stream)), "fairy_cattention")


def fairy_cgemv_rope(L, x_re, x_im, xdtype, batch, ldx, y_re, y_im, ldy, positions, head_dim, base, stream=None):
    _check(lib().fairy_cgemv_rope(ctypes.byref(L), _ptr(x_re), _ptr(x_im), xdtype, batch, ldx, _ptr(y_re),
                                  _ptr(y_im), ldy, _ptr(positions), head_dim, float(base), _stream(stream)),
           "fairy_cgemv_rope")


def fairy_cgemm_rope(L, x_re, x_im, xdtype, M, ldx, y_re, y_im, ldy, algo, positions, head_dim, base, stream=None):
    _check(lib().fairy_cgemm_rope(ctypes.byref(L), _ptr(x_re), _ptr(x_im), xdtype, M, ldx, _ptr(y_re), _ptr(y_im),
                                  ldy, algo, _ptr(positions), head_dim, float(base), _stream(stream)),
           "fairy_cgemm_rope")


def fairy_cgemv_lut_workspace_bytes(L) -> int:
    return lib().fairy_cgemv_lut_workspace_bytes(ctypes.byref(L))


def fairy_cgemv_lut(L, x_re, x_im, xdtype, y_re, y_im, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().fairy_cgemv_lut(ctypes.byref(L), _ptr(x_re), _ptr(x_im), xdtype, _ptr(y_re), _ptr(y_im),
                                 _ptr(workspace), workspace_bytes, _stream(stream)), "fairy_cgemv_lut")
