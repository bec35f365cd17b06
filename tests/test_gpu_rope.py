"""GPU parity of the rotary position encoding fused into the GEMV / GEMM
epilogue: the oracle's layer output, rotated by the oracle's rope, against
fairy_cgemv_rope / fairy_cgemm_rope (relative L2 <= 1e-5, the GEMV bound;
the rotation itself is evaluated in fp64)."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, layer_from_codes, log, rel_l2, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5


def inputs(B, m, xdtype, seed):
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((B, m), seed)
        return rb, ib, synth.bf16_to_f32(rb), synth.bf16_to_f32(ib)
    if xdtype == F.FAIRY_F32:
        xr, xi = synth.complex_gaussian((B, m), 1.0, seed)
        return xr, xi, xr, xi
    xr, xi = synth.int8_uniform((B, m), seed)
    return xr, xi, xr.astype(np.float64), xi.astype(np.float64)


def run(layer, xr, xi, xdtype, B, pos, head_dim, base, gemm=False, algo=F.FAIRY_ALGO_AUTO):
    t = torch()
    n, m = layer.n, layer.m
    yr = t.empty((B, n), dtype=t.float32, device="cuda")
    yi = t.empty_like(yr)
    p = dev(np.asarray(pos, np.int32))
    if gemm:
        F.fairy_cgemm_rope(layer.desc, dev(xr), dev(xi), xdtype, B, m, yr, yi, n, algo, p, head_dim, base)
    else:
        F.fairy_cgemv_rope(layer.desc, dev(xr), dev(xi), xdtype, B, m, yr, yi, n, p, head_dim, base)
    t.cuda.synchronize()
    return host(yr), host(yi)


CASES = [
    # (S, has_conj, n, m, B, xdtype, head_dim)
    (2, True, 256, 512, 3, F.FAIRY_BF16, 64),      # one row per wave, P = 4
    (2, True, 128, 2048, 5, F.FAIRY_F32, 32),
    (3, True, 100, 256, 2, F.FAIRY_BF16, 50),      # P = 6: the generic kernel; head_dim not a power of 2
    (1, False, 64, 64, 4, F.FAIRY_BF16, 16),       # short rows
    (2, True, 96, 512, 3, F.FAIRY_I8, 64),
]


@pytest.mark.parametrize("S,hc,n,m,B,xdtype,hd", CASES)
def test_cgemv_rope(S, hc, n, m, B, xdtype, hd):
    log(f"cgemv_rope S={S} conj={hc} n={n} m={m} B={B} dt={xdtype} hd={hd}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 31 + n)
    scales = synth.random_scales(P, 37 + m)
    layer = layer_from_codes(codes, scales, S, hc)
    xr, xi, fr, fi = inputs(B, m, xdtype, 41 + B)
    pos = synth.rng(43).integers(0, 4096, B)
    yr, yi = run(layer, xr, xi, xdtype, B, pos, hd, 10000.0)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, fr, fi)
    wr, wi = oracle.rope(wr, wi, pos, hd, 10000.0)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("S,hc,n,m,M,xdtype,algo", [
    (2, True, 130, 512, 70, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA),
    (3, True, 64, 256, 33, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA),     # two passes: the rotation only on the last
    (3, False, 50, 192, 20, F.FAIRY_I8, F.FAIRY_ALGO_MFMA),      # P = 3: passes of 2 and 1
    (2, True, 64, 128, 40, F.FAIRY_F32, F.FAIRY_ALGO_VALU),
])
def test_cgemm_rope(S, hc, n, m, M, xdtype, algo):
    log(f"cgemm_rope S={S} conj={hc} n={n} m={m} M={M} dt={xdtype} algo={algo}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 51 + n)
    scales = synth.random_scales(P, 53 + m)
    layer = layer_from_codes(codes, scales, S, hc)
    xr, xi, fr, fi = inputs(M, m, xdtype, 57)
    pos = np.arange(M) + 100      # consecutive token positions
    yr, yi = run(layer, xr, xi, xdtype, M, pos, 32, 500.0, gemm=True, algo=algo)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, fr, fi)
    wr, wi = oracle.rope(wr, wi, pos, 32, 500.0)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


def test_rope_position_zero_equals_plain_gemv():
    S, n, m, B = 2, 64, 256, 2
    codes = synth.random_codes((4, n, m), 61)
    scales = synth.random_scales(4, 62)
    layer = layer_from_codes(codes, scales, S, True)
    xr, xi, _, _ = inputs(B, m, F.FAIRY_BF16, 63)
    yr, yi = run(layer, xr, xi, F.FAIRY_BF16, B, [0, 0], 64, 10000.0)
    from tests._gpu import run_gemv
    pr, pi, _ = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_BF16, B)
    assert np.array_equal(yr, pr) and np.array_equal(yi, pi)
