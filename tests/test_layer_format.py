"""Host-side checks of the serialised quantised-layer format and of the
conversion entry points' argument validation (no device is touched).

The format is libfairy's own (the pages define none; their deployment notes
only ask for a complex storage format the device supports, with real and
imaginary parts kept apart): the buffers below are built from the byte
layout written in include/fairy.h, not from the library.
"""
import struct

import pytest

from bit_complex_weight_amd import fairy as F

A = 1 << 20          # a fake, 256-byte aligned device address: validation fails before any use


def header(n, m, S, conj, P=None, layout=F.FAIRY_LAYOUT_TILED64, version=1, magic=b"FAIRYQL1", hb=None,
           packed_bytes=None):
    P = S * (1 + conj) if P is None else P
    hb = ((64 + 8 * P + 63) // 64) * 64 if hb is None else hb
    G = (m + 63) // 64
    pb = n * G * P * 16 if packed_bytes is None else packed_bytes
    h = magic + struct.pack("<IIqqiiiiQQ", version, hb, n, m, S, conj, layout, P, pb, 0)
    assert len(h) == 64
    scales = struct.pack("<" + "f" * (2 * P), *[0.5 + i for i in range(2 * P)])
    body = h + scales + b"\0" * (hb - 64 - 8 * P)
    return bytearray(body + bytes(range(256)) * (pb // 256) + bytes(pb % 256))


def test_file_bytes():
    # 2048 x 2048, S = 2 widely-linear: header 64 + 32 -> 128 bytes, 4 MiB of words
    assert F.fairy_layer_file_bytes(2048, 2048, 2, 1) == 128 + 4 * 1024 * 1024
    # one plane: 64 + 8 -> 128
    assert F.fairy_layer_file_bytes(256, 256, 1, 0) == 128 + 256 * 4 * 16
    # 8 stages with conj: P = 16, 64 + 128 = 192
    assert F.fairy_layer_file_bytes(3, 80, 8, 1) == 192 + 3 * 2 * 16 * 16
    assert F.fairy_layer_file_bytes(0, 64, 1, 0) == 0
    assert F.fairy_layer_file_bytes(4, 72, 1, 0) == 0        # m % 16
    assert F.fairy_layer_file_bytes(4, 64, 9, 0) == 0
    assert F.fairy_layer_file_bytes(4, 64, 1, 2) == 0


@pytest.mark.parametrize("n,m,S,conj", [(2048, 2048, 2, 1), (37, 80, 3, 1), (256, 256, 1, 0), (5, 16, 8, 1)])
def test_read_info(n, m, S, conj):
    buf = header(n, m, S, conj)
    info = F.fairy_layer_read_info(buf)
    P = S * (1 + conj)
    assert (info.n, info.m, info.stages, info.has_conj, info.layout, info.planes) == (
        n, m, S, conj, F.FAIRY_LAYOUT_TILED64, P)
    assert info.packed_bytes == F.fairy_packed_words(n, m, P, F.FAIRY_LAYOUT_TILED64) * 4
    assert info.header_bytes == ((64 + 8 * P + 63) // 64) * 64
    assert len(buf) == F.fairy_layer_file_bytes(n, m, S, conj)


@pytest.mark.parametrize("mutate,want", [
    (dict(magic=b"FAIRYQL2"), F.FAIRY_ERR_INVALID_ARG),
    (dict(version=2), F.FAIRY_ERR_UNSUPPORTED),
    (dict(layout=F.FAIRY_LAYOUT_ROW16), F.FAIRY_ERR_UNSUPPORTED),
    (dict(P=3), F.FAIRY_ERR_INVALID_ARG),                 # planes != S (1 + conj)
    (dict(hb=64), F.FAIRY_ERR_INVALID_ARG),
    (dict(packed_bytes=16), F.FAIRY_ERR_INVALID_ARG),
])
def test_read_info_rejects(mutate, want):
    buf = header(37, 80, 2, 1, **mutate)
    with pytest.raises(F.FairyError) as e:
        F.fairy_layer_read_info(buf)
    assert e.value.status == want


def test_read_info_truncated():
    buf = header(37, 80, 2, 1)
    for cut in (0, 10, 63, len(buf) - 1):
        with pytest.raises(F.FairyError) as e:
            F.fairy_layer_read_info(bytes(buf[:cut]))
        assert e.value.status == F.FAIRY_ERR_INVALID_ARG


def test_quantize_workspace_bytes():
    # real: 2S code planes + U's and W's buckets (S x 16 copies of 514 uint64
    # each), each region 256-aligned; U and W are formed inside PhaseQuant
    n, m, S = 2048, 2048, 2
    pq = S * 16 * 514 * 8
    want = 2 * S * n * m + ((2 * pq + 255) // 256) * 256
    assert F.fairy_quantize_workspace_bytes(n, m, S, 1) == want
    assert F.fairy_quantize_workspace_bytes(n, m, S, 0) == S * n * m + ((pq + 255) // 256) * 256
    assert F.fairy_quantize_workspace_bytes(0, m, S, 1) == 0
    assert F.fairy_quantize_workspace_bytes(n, m, 9, 1) == 0
    assert F.fairy_quantize_workspace_bytes(1 << 16, 1 << 16, 1, 0) == 0     # n*m >= 2^32


def _raw(name, *args):
    return getattr(F.lib(), name)(*args)


def test_quantize_validation():
    ws = F.fairy_quantize_workspace_bytes(64, 64, 2, 1)
    assert _raw("fairy_quantize_real", None, 64, 64, 2, A, A, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_real", A, 0, 64, 2, A, A, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_real", A, 64, 64, 0, A, A, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_real", A, 64, 64, 2, None, A, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_real", A, 64, 64, 2, A + 4, A, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_real", A, 64, 72, 2, A, A, A, 1 << 30, None) == F.FAIRY_ERR_UNSUPPORTED
    assert _raw("fairy_quantize_real", A, 64, 64, 2, A, A, A, ws - 1, None) == F.FAIRY_ERR_WORKSPACE
    assert _raw("fairy_quantize_real", A, 64, 64, 2, A, A, A + 16, ws, None) == F.FAIRY_ERR_WORKSPACE
    assert _raw("fairy_quantize_real", A, 64, 64, 2, A, A, None, ws, None) == F.FAIRY_ERR_WORKSPACE
    wc = F.fairy_quantize_workspace_bytes(64, 64, 2, 0)
    assert _raw("fairy_quantize_complex", A, None, 64, 64, 2, A, A, A, wc, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_quantize_complex", A, A, 64, 64, 2, A, A, A, wc - 1, None) == F.FAIRY_ERR_WORKSPACE


def test_save_load_validation():
    L = F.make_clinear(37, 80, 2, 1, A, A)
    small = bytearray(16)
    assert _raw("fairy_layer_save", None, F._host_buf(small)[0], 16, None) == F.FAIRY_ERR_INVALID_ARG
    import ctypes
    assert _raw("fairy_layer_save", ctypes.byref(L), F._host_buf(small)[0], 16, None) == F.FAIRY_ERR_WORKSPACE
    Lr = F.make_clinear(37, 80, 2, 1, A, A, layout=F.FAIRY_LAYOUT_ROW16)
    assert _raw("fairy_layer_save", ctypes.byref(Lr), F._host_buf(small)[0], 16, None) == F.FAIRY_ERR_UNSUPPORTED
    buf = header(37, 80, 2, 1)
    addr, size = F._host_buf(buf)
    assert _raw("fairy_layer_load", addr, size, None, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_layer_load", addr, size, A + 4, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert _raw("fairy_layer_load", addr, 40, A, A, None) == F.FAIRY_ERR_INVALID_ARG


def test_cattention_validation():
    """Argument checks of fairy_cattention (all fail before any device work)."""
    f = F.lib().fairy_cattention
    ok = dict(q=A, k=A, v=A, o=A, dt=F.FAIRY_BF16, h=2, sq=64, sk=64, d=64, scale=0.1, causal=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["q"], a["k"], a["k"], a["v"], a["v"], a["dt"], a["h"], a["sq"], a["sk"], a["d"],
                 a["scale"], a["causal"], a["o"], a["o"], None)

    assert call(q=None) == F.FAIRY_ERR_INVALID_ARG
    assert call(k=A + 8) == F.FAIRY_ERR_INVALID_ARG
    assert call(o=None) == F.FAIRY_ERR_INVALID_ARG
    assert call(h=0) == F.FAIRY_ERR_INVALID_ARG
    assert call(h=70000) == F.FAIRY_ERR_INVALID_ARG
    assert call(sq=0) == F.FAIRY_ERR_INVALID_ARG
    assert call(sk=0) == F.FAIRY_ERR_INVALID_ARG
    assert call(causal=2) == F.FAIRY_ERR_INVALID_ARG
    assert call(causal=1, sq=65, sk=64) == F.FAIRY_ERR_INVALID_ARG     # causal needs sk >= sq
    assert call(scale=float("nan")) == F.FAIRY_ERR_INVALID_ARG
    assert call(dt=7) == F.FAIRY_ERR_INVALID_ARG
    assert call(dt=F.FAIRY_F32) == F.FAIRY_ERR_UNSUPPORTED
    assert call(dt=F.FAIRY_I8) == F.FAIRY_ERR_UNSUPPORTED
    assert call(d=48) == F.FAIRY_ERR_UNSUPPORTED
    assert call(d=256) == F.FAIRY_ERR_UNSUPPORTED


def test_rope_validation():
    import ctypes
    L = F.make_clinear(64, 64, 2, 1, A, A)
    f = F.lib().fairy_cgemv_rope
    g = F.lib().fairy_cgemm_rope
    r = ctypes.byref(L)
    assert f(r, A, A, F.FAIRY_BF16, 1, 64, A, A, 64, None, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(r, A, A, F.FAIRY_BF16, 1, 64, A, A, 64, A + 2, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(r, A, A, F.FAIRY_BF16, 1, 64, A, A, 64, A, 0, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(r, A, A, F.FAIRY_BF16, 1, 64, A, A, 64, A, 64, 0.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(r, A, A, F.FAIRY_BF16, 1, 64, A, A, 64, A, 64, float("inf"), None) == F.FAIRY_ERR_INVALID_ARG
    assert f(r, A, A, F.FAIRY_BF16, 65, 64, A, A, 64, A, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert g(r, A, A, F.FAIRY_BF16, 0, 64, A, A, 64, F.FAIRY_ALGO_AUTO, A, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert g(r, A, A, F.FAIRY_BF16, 8, 64, A, A, 64, 9, A, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
    assert g(r, A, A, F.FAIRY_F32, 8, 64, A, A, 64, F.FAIRY_ALGO_MFMA, A, 64, 10000.0, None) == F.FAIRY_ERR_UNSUPPORTED
    assert g(r, A, A, F.FAIRY_BF16, 8, 64, A, A, 64, F.FAIRY_ALGO_AUTO, None, 64, 10000.0, None) == F.FAIRY_ERR_INVALID_ARG
