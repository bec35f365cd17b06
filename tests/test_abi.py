"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/fairy.h declares,
keep the oracle out of the product library, and reject invalid arguments on
the host with the documented status before any launch (so these calls never
reach the device).
"""
import ctypes
import os
import re
import subprocess

import pytest

from bit_complex_weight_amd import fairy as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fairy.h")

A = 0x10000  # a 16-byte aligned fake device address: never dereferenced here


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fairy_[a-z0-9_]+)\s*\(", txt)))


def exported_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_library_loads():
    assert F.fairy_abi_version() == 1


def test_every_declared_entry_point_is_exported():
    decl = declared_functions()
    assert len(decl) >= 12, decl
    syms = exported_symbols()
    missing = [d for d in decl if d not in syms]
    assert not missing, missing


def test_oracle_not_linked_into_product():
    syms = exported_symbols()
    assert not any(s.startswith("orc_") for s in syms)
    out = subprocess.run(["ldd", F.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out


def test_status_strings():
    seen = set()
    for s in range(5):
        t = F.status_string(s)
        assert t and t not in seen
        seen.add(t)
    assert "UNKNOWN" in F.status_string(99)


def test_packed_words():
    assert F.fairy_packed_words(2048, 2048, 4, F.FAIRY_LAYOUT_TILED64) == 2048 * 32 * 4 * 4
    assert F.fairy_packed_words(2048, 5504, 4, F.FAIRY_LAYOUT_TILED64) == 2048 * 86 * 4 * 4
    assert F.fairy_packed_words(256, 256, 1, F.FAIRY_LAYOUT_ROW16) == 256 * 16
    assert F.fairy_packed_words(10, 80, 2, F.FAIRY_LAYOUT_TILED64) == 10 * 2 * 2 * 4   # padded to 128 cols
    assert F.fairy_packed_words(10, 24, 1, F.FAIRY_LAYOUT_ROW16) == -1                 # m % 16
    assert F.fairy_packed_words(0, 16, 1, 0) == -1
    assert F.fairy_packed_words(1, 16, 17, 0) == -1
    assert F.fairy_packed_words(1, 16, 1, 7) == -1


def test_workspace_sizes():
    assert F.fairy_phasequant_workspace_bytes(1000, 2) == 2 * 16 * 514 * 8
    assert F.fairy_phasequant_workspace_bytes(0, 2) == 0
    assert F.fairy_phasequant_workspace_bytes(10, 9) == 0
    assert F.fairy_phasequant_workspace_bytes(1 << 32, 1) == 0


def test_cgemm_workspace_sizes():
    """The matrix-core GEMM asks for a K-split workspace only where its
    64-row x 64-token blocks would leave CUs idle: splits x 2 x M x n floats."""
    L = F.make_clinear(2048, 2048, 2, 1, A, A)                   # P = 4: 32 row blocks
    ws = lambda M, dt, algo: F.fairy_cgemm_workspace_bytes(L, M, dt, algo)
    # bf16: 16 chunks of 128 columns; 32 blocks -> 8 splits of 2 chunks
    assert ws(16, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) == 8 * 2 * 16 * 2048 * 4
    assert ws(64, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) == 8 * 2 * 64 * 2048 * 4
    # int8: 8 chunks of 256 columns -> 8 splits of 1
    assert ws(64, F.FAIRY_I8, F.FAIRY_ALGO_MFMA) == 8 * 2 * 64 * 2048 * 4
    # 3 token blocks -> 96 blocks -> 3 splits of 6 chunks (bf16)
    assert ws(150, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) == 3 * 2 * 150 * 2048 * 4
    # enough blocks, the VALU path, AUTO below its matrix-core threshold, fp32: none
    assert ws(256, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) == 0          # 128 blocks
    assert ws(2048, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) == 0
    assert ws(16, F.FAIRY_BF16, F.FAIRY_ALGO_VALU) == 0
    assert ws(8, F.FAIRY_BF16, F.FAIRY_ALGO_AUTO) == 0
    assert ws(16, F.FAIRY_BF16, F.FAIRY_ALGO_AUTO) == 8 * 2 * 16 * 2048 * 4
    assert ws(64, F.FAIRY_F32, F.FAIRY_ALGO_MFMA) == 0
    # plane counts that need several passes: none
    assert F.fairy_cgemm_workspace_bytes(F.make_clinear(2048, 2048, 3, 1, A, A), 16, F.FAIRY_BF16,
                                         F.FAIRY_ALGO_MFMA) == 0
    # a short row (one chunk) cannot be split
    assert F.fairy_cgemm_workspace_bytes(F.make_clinear(64, 128, 1, 0, A, A), 8, F.FAIRY_BF16,
                                         F.FAIRY_ALGO_MFMA) == 0


def status_of(fn, *args):
    return fn(*args)


L_ = F.lib()


def test_real_to_complex_validation():
    f = L_.fairy_real_to_complex
    assert f(None, 2, 2, A, A, A, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, 0, 2, A, A, A, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, 2, -1, A, A, A, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A + 1, 2, 2, A, A, A, A, None) == F.FAIRY_ERR_INVALID_ARG


def test_phasequant_validation():
    f = L_.fairy_phasequant
    ws = F.fairy_phasequant_workspace_bytes(100, 2)
    assert f(None, A, 100, 2, A, A, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 0, 2, A, A, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 1 << 32, 2, A, A, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 0, A, A, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 9, A, A, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, A, A + 2, None, None, A, ws, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, A, A, None, None, None, ws, None) == F.FAIRY_ERR_WORKSPACE
    assert f(A, A, 100, 2, A, A, None, None, A, ws - 1, None) == F.FAIRY_ERR_WORKSPACE
    assert f(A, A, 100, 2, A, A, None, None, A + 4, ws, None) == F.FAIRY_ERR_WORKSPACE


def test_pack_validation():
    for f in (L_.fairy_pack, L_.fairy_unpack):
        assert f(None, 1, 4, 16, 0, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A, 0, 4, 16, 0, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A, 17, 4, 16, 0, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A, 1, 0, 16, 0, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A, 1, 4, 16, 2, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A + 8, 1, 4, 16, 0, A, None) == F.FAIRY_ERR_INVALID_ARG
        assert f(A, 1, 4, 24, 0, A, None) == F.FAIRY_ERR_UNSUPPORTED
        assert f(A, 1, 4, 24, 1, A, None) == F.FAIRY_ERR_UNSUPPORTED


def layer(**kw):
    d = dict(n=64, m=64, stages=2, has_conj=1, layout=F.FAIRY_LAYOUT_TILED64, packed=A, scales=A)
    d.update(kw)
    return F.fairy_clinear(d["n"], d["m"], d["stages"], d["has_conj"], d["layout"], d["packed"], d["scales"])


def gemv(Lr, xr=A, xi=A, dt=F.FAIRY_BF16, B=1, ldx=64, yr=A, yi=A, ldy=64, acc=None):
    return L_.fairy_cgemv(ctypes.byref(Lr) if Lr is not None else None, xr, xi, dt, B, ldx, yr, yi, ldy, acc,
                          None, 0, None)


@pytest.mark.parametrize("kw,call,want", [
    ({}, dict(B=0), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(B=65), F.FAIRY_ERR_INVALID_ARG),
    ({"n": 0}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"stages": 0}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"stages": 9}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"has_conj": 2}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"layout": 5}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"packed": None}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"scales": None}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({"packed": A + 4}, {}, F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(xr=None), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(xi=A + 8), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(dt=3), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(ldx=48), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(ldx=72), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(ldy=63), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(yr=None), F.FAIRY_ERR_INVALID_ARG),
    ({}, dict(acc=A), F.FAIRY_ERR_INVALID_ARG),            # acc only with I8
    ({"layout": F.FAIRY_LAYOUT_ROW16}, {}, F.FAIRY_ERR_UNSUPPORTED),
    ({"m": 72}, dict(ldx=80), F.FAIRY_ERR_UNSUPPORTED),     # m % 16
    ({"m": 16400}, dict(ldx=16400), F.FAIRY_ERR_UNSUPPORTED),
    ({"m": 14592}, dict(ldx=14592), F.FAIRY_ERR_UNSUPPORTED),  # bf16 activations beyond 64 KiB of LDS
    ({"m": 7744}, dict(ldx=7744, dt=F.FAIRY_F32), F.FAIRY_ERR_UNSUPPORTED),
    ({"m": 26176}, dict(ldx=26176, dt=F.FAIRY_I8), F.FAIRY_ERR_UNSUPPORTED),
])
def test_cgemv_validation(kw, call, want):
    assert gemv(layer(**kw), **call) == want


def test_cgemv_null_layer():
    assert gemv(None) == F.FAIRY_ERR_INVALID_ARG


def test_cgemm_validation():
    f = L_.fairy_cgemm
    Lr = layer()
    args = lambda M=8, dt=F.FAIRY_BF16, algo=0, acc=None: (ctypes.byref(Lr), A, A, dt, M, 64, A, A, 64, acc, algo,
                                                          None, 0, None)
    assert f(*args(M=0)) == F.FAIRY_ERR_INVALID_ARG
    assert f(*args(algo=3)) == F.FAIRY_ERR_INVALID_ARG
    assert f(*args(acc=A)) == F.FAIRY_ERR_INVALID_ARG
    assert f(*args(dt=F.FAIRY_F32, algo=F.FAIRY_ALGO_MFMA)) == F.FAIRY_ERR_UNSUPPORTED
    # beyond the staged-activation width: unsupported on the VALU path (and
    # on AUTO below its matrix-core threshold); the matrix-core path streams
    Lw = layer(m=16384)
    wide = lambda M, algo: f(ctypes.byref(Lw), A, A, F.FAIRY_BF16, M, 16384, A, A, 64, None, algo, None, 0, None)
    assert wide(8, F.FAIRY_ALGO_VALU) == F.FAIRY_ERR_UNSUPPORTED
    assert wide(8, F.FAIRY_ALGO_AUTO) == F.FAIRY_ERR_UNSUPPORTED
    # the optional K-split workspace: a given one must be large enough and aligned
    Lb = layer(n=2048, m=2048)
    need = F.fairy_cgemm_workspace_bytes(Lb, 16, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA)
    assert need > 0
    split = lambda w, wb: f(ctypes.byref(Lb), A, A, F.FAIRY_BF16, 16, 2048, A, A, 2048, None, F.FAIRY_ALGO_MFMA, w, wb,
                            None)
    assert split(A, need - 1) == F.FAIRY_ERR_WORKSPACE
    assert split(A + 4, need) == F.FAIRY_ERR_WORKSPACE


def test_cgemv_lut_validation():
    f, ws = L_.fairy_cgemv_lut, L_.fairy_cgemv_lut_workspace_bytes
    big = layer(n=2048, m=2048)
    need = ws(ctypes.byref(big))
    assert need > 0 and need % (8 * 2048) == 0   # fp32 (re, im) partial rows per column chunk
    assert ws(ctypes.byref(layer(m=16, stages=1, has_conj=0))) == 0   # one 16-byte unit per row: one chunk
    assert ws(ctypes.byref(layer(n=0))) == 0
    assert ws(None) == 0

    def call(Lr, dt=F.FAIRY_BF16, xr=A, w=None, wb=0):
        return f(ctypes.byref(Lr) if Lr is not None else None, xr, A, dt, A, A, w, wb, None)

    assert call(None) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(n=0)) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(stages=9)) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(packed=0)) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(), xr=A + 2) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(), dt=7) == F.FAIRY_ERR_INVALID_ARG
    assert call(layer(), dt=F.FAIRY_I8) == F.FAIRY_ERR_UNSUPPORTED
    assert call(layer(m=40)) == F.FAIRY_ERR_UNSUPPORTED
    assert call(layer(layout=F.FAIRY_LAYOUT_ROW16)) == F.FAIRY_ERR_UNSUPPORTED
    assert call(big) == F.FAIRY_ERR_WORKSPACE
    assert call(big, w=A, wb=need - 1) == F.FAIRY_ERR_WORKSPACE
    assert call(big, w=A + 4, wb=need) == F.FAIRY_ERR_WORKSPACE


def test_python_binding_rejects_host_buffers():
    import numpy as np
    with pytest.raises(TypeError):
        F._ptr(np.zeros(4))


def test_cgemv_group_validation():
    """Grouped GEMV: 1..8 layers sharing m, stages and the conjugate branch;
    every layer checked as fairy_cgemv checks it; host arrays required."""
    f = L_.fairy_cgemv_group
    P = ctypes.c_void_p

    def call(layers, batch=1, ldy=None, yr=None, yi=None, dt=F.FAIRY_BF16, ldx=2048):
        k = len(layers)
        arr = (F.fairy_clinear * max(k, 1))(*layers) if k else None
        yr = yr if yr is not None else (P * max(k, 1))(*([A] * max(k, 1)))
        yi = yi if yi is not None else (P * max(k, 1))(*([A] * max(k, 1)))
        ld = ldy if ldy is not None else (ctypes.c_int64 * max(k, 1))(*[l.n for l in layers] or [1])
        return f(arr, k, A, A, dt, batch, ldx, ctypes.cast(yr, P) if yr else None,
                 ctypes.cast(yi, P) if yi else None, ctypes.cast(ld, P) if ld else None, None)

    q = F.make_clinear(2048, 2048, 2, 1, A, A)
    gate = F.make_clinear(5504, 2048, 2, 1, A, A)
    assert call([]) == F.FAIRY_ERR_INVALID_ARG                          # count 0
    assert call([q] * 9) == F.FAIRY_ERR_INVALID_ARG                     # count > 8
    assert call([q, gate], batch=0) == F.FAIRY_ERR_INVALID_ARG
    assert call([q, gate], batch=65) == F.FAIRY_ERR_INVALID_ARG
    assert call([q, F.make_clinear(2048, 4096, 2, 1, A, A)]) == F.FAIRY_ERR_INVALID_ARG   # m differs
    assert call([q, F.make_clinear(2048, 2048, 1, 1, A, A)]) == F.FAIRY_ERR_INVALID_ARG   # stages differ
    assert call([q, F.make_clinear(2048, 2048, 2, 0, A, A)]) == F.FAIRY_ERR_INVALID_ARG   # conj differs
    assert call([q, F.make_clinear(2048, 2048, 2, 1, A + 4, A)]) == F.FAIRY_ERR_INVALID_ARG  # misaligned words
    assert call([q, q], ldy=(ctypes.c_int64 * 2)(2048, 2047)) == F.FAIRY_ERR_INVALID_ARG    # ldy < n
    assert call([q, q], yr=(P * 2)(A, None)) == F.FAIRY_ERR_INVALID_ARG                    # null output
    assert f(None, 1, A, A, F.FAIRY_BF16, 1, 2048, A, A, A, None) == F.FAIRY_ERR_INVALID_ARG
    arr = (F.fairy_clinear * 1)(q)
    assert f(arr, 1, A, A, F.FAIRY_BF16, 1, 2048, None, A, A, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(arr, 1, A, A, F.FAIRY_BF16, 1, 2048, A, A, None, None) == F.FAIRY_ERR_INVALID_ARG
    # same width rules as fairy_cgemv: m % 16, the staged-activation limit
    assert call([F.make_clinear(64, 24, 1, 0, A, A)], ldx=32) == F.FAIRY_ERR_UNSUPPORTED
    wide = F.make_clinear(64, 16384, 1, 0, A, A)
    assert call([wide], ldx=16384) == F.FAIRY_ERR_UNSUPPORTED


def test_phasequant_noalloc_validation():
    """The allocation-free PhaseQuant checks its arguments as fairy_phasequant
    does (no workspace argument) before any HIP call."""
    f = L_.fairy_phasequant_noalloc
    assert f(None, A, 100, 2, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, None, 100, 2, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, None, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, A, None, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 0, 2, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 1 << 32, 2, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 0, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 9, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A + 2, A, 100, 2, A, A, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, A, A + 2, None, None, None) == F.FAIRY_ERR_INVALID_ARG
    assert f(A, A, 100, 2, A, A, A + 1, None, None) == F.FAIRY_ERR_INVALID_ARG
