"""GPU parity of the table-lookup GEMV (fairy_cgemv_lut) against the CPU oracle.

The lookup path computes the same y = sum U_k x + sum W_k conj(x) as the
direct decode, so it is held to the same bar: relative L2 error <= 1e-5
against the fp64 oracle on the same (bf16- or fp32-valued) inputs.  Cases
cover ragged rows (blocks of 64, 128 or 256 rows), ragged column groups,
plane counts 1..16, column chunks that do not divide a row, widths beyond
the direct path's LDS staging limit and the full layer shapes.
"""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, layer_from_codes, log, rel_l2, run_gemv, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5


def run_lut(layer, x_re, x_im, xdtype):
    t = torch()
    n = layer.n
    y_re = t.empty(n, dtype=t.float32, device="cuda")
    y_im = t.empty(n, dtype=t.float32, device="cuda")
    wsb = F.fairy_cgemv_lut_workspace_bytes(layer.desc)
    ws = t.empty(max(wsb, 1), dtype=t.uint8, device="cuda") if wsb else None
    F.fairy_cgemv_lut(layer.desc, x_re, x_im, xdtype, y_re, y_im, ws, wsb)
    t.cuda.synchronize()
    return host(y_re), host(y_im)


def inputs(m, xdtype, seed):
    """Device activations and their exact float64 values."""
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((1, m), seed)
        return dev(rb[0]), dev(ib[0]), synth.bf16_to_f32(rb[0]), synth.bf16_to_f32(ib[0])
    xr, xi = synth.complex_gaussian((1, m), 1.0, seed)
    return dev(xr[0]), dev(xi[0]), xr[0], xi[0]


def check(S, hc, n, m, xdtype, seed):
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), seed)
    scales = synth.random_scales(P, seed + 1)
    layer = layer_from_codes(codes, scales, S, hc)
    dxr, dxi, xr, xi = inputs(m, xdtype, seed + 2)
    yr, yi = run_lut(layer, dxr, dxi, xdtype)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr[None].astype(np.float64), xi[None].astype(np.float64))
    err = rel_l2(yr + 1j * yi, wr[0] + 1j * wi[0])
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
    return layer, (dxr, dxi), (yr, yi)


CASES = [
    # (S, has_conj, n, m)
    (1, False, 1, 16),         # one unit per row, one row
    (1, True, 5, 64),
    (2, True, 37, 80),         # ragged rows and a half-empty column group
    (3, True, 64, 208),        # P = 6
    (2, False, 100, 1024),
    (4, True, 9, 128),         # P = 8
    (8, True, 3, 64),          # P = 16
    (7, False, 33, 64),        # P = 7: chunks straddle column groups
    (2, True, 130, 2048),
    (2, True, 300, 5504),      # 344 units per row: a partial last chunk
    (1, True, 257, 4112),      # ragged last group, P = 2
    (3, False, 1000, 336),     # many rows, few units
]


@pytest.mark.parametrize("S,hc,n,m", CASES)
@pytest.mark.parametrize("xdtype", [F.FAIRY_BF16, F.FAIRY_F32])
def test_lut_random_codes(S, hc, n, m, xdtype):
    log(f"lut S={S} conj={hc} n={n} m={m} dt={xdtype}")
    check(S, hc, n, m, xdtype, 13 * n + m + S)


@pytest.mark.parametrize("xdtype,m", [(F.FAIRY_BF16, 16384), (F.FAIRY_F32, 8192)])
def test_lut_beyond_staging_limit(xdtype, m):
    """Widths the direct path rejects (activations do not fit its LDS
    staging) are served by the lookup path."""
    log(f"lut wide m={m} dt={xdtype}")
    check(2, True, 70, m, xdtype, 900 + m)


def test_lut_matches_direct_and_is_deterministic():
    log("lut vs direct decode, 2048x2048 S=2 widely-linear, bf16")
    layer, (dxr, dxi), (yr, yi) = check(2, True, 2048, 2048, F.FAIRY_BF16, 31)
    again = run_lut(layer, dxr, dxi, F.FAIRY_BF16)
    assert np.array_equal(again[0], yr) and np.array_equal(again[1], yi)
    dr, di, _ = run_gemv(layer, dxr[None], dxi[None], F.FAIRY_BF16, 1)
    assert rel_l2(yr + 1j * yi, dr[0] + 1j * di[0]) <= 2 * TOL


@pytest.mark.parametrize("n,m", [(2048, 2048), (5504, 2048), (2048, 5504)])
def test_lut_full_layer_shapes(n, m):
    """The decode-step layer shapes (complex rows x columns of the 4096- and
    11008-wide real layers, S = 2 widely-linear), every output checked."""
    log(f"lut full shape {n}x{m} S=2")
    check(2, True, n, m, F.FAIRY_BF16, 500 + n + m)


def test_lut_rejects_small_workspace():
    codes = synth.random_codes((4, 2048, 2048), 3)
    layer = layer_from_codes(codes, synth.random_scales(4, 4), 2, True)
    t = torch()
    wsb = F.fairy_cgemv_lut_workspace_bytes(layer.desc)
    assert wsb > 0
    y = t.empty(2048, dtype=t.float32, device="cuda")
    x = t.zeros(2048, dtype=t.int16, device="cuda")
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    with pytest.raises(F.FairyError) as e:
        F.fairy_cgemv_lut(layer.desc, x, x, F.FAIRY_BF16, y, y, ws, wsb - 1)
    assert e.value.status == F.FAIRY_ERR_WORKSPACE
