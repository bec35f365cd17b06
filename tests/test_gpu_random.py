"""Seeded random-shape parity sweeps: GEMV, GEMM and attention configurations
drawn from the argument space (plane counts, ragged rows, columns and
tokens, every activation type and algorithm, with and without the GEMM
workspace), each compared with the fp64 / exact oracle to the same bounds
as the fixed cases: <= 1e-5 relative L2 for float outputs (attention
included), int32 accumulators exact."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, layer_from_codes, log, rel_l2, run_gemv, torch, host

pytestmark = pytest.mark.gpu
TOL = 1e-5
DTYPES = {F.FAIRY_BF16: "bf16", F.FAIRY_F32: "f32", F.FAIRY_I8: "i8"}


def activations(xdtype, B, m, seed):
    """(device re, device im, fp64 re, fp64 im) of the given type."""
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((B, m), seed)
        return dev(rb), dev(ib), synth.bf16_to_f32(rb).astype(np.float64), synth.bf16_to_f32(ib).astype(np.float64)
    if xdtype == F.FAIRY_F32:
        xr, xi = synth.complex_gaussian((B, m), 1.0, seed)
        return dev(xr), dev(xi), xr.astype(np.float64), xi.astype(np.float64)
    xr, xi = synth.int8_uniform((B, m), seed)
    return dev(xr), dev(xi), xr.astype(np.float64), xi.astype(np.float64)


def gemv_case(i):
    g = synth.rng(7000 + i)
    S = int(g.integers(1, 5))
    hc = bool(g.integers(0, 2))
    n = int(g.integers(1, 261))
    m = 16 * int(g.integers(1, 161))
    B = int(g.choice([1, 1, 2, 3, 4, 5, 8, 13, 16, 33, 64]))
    if B > 16:
        n = min(n, 64)
    xdtype = int(g.choice(list(DTYPES)))
    return S, hc, n, m, B, xdtype


@pytest.mark.parametrize("i", range(60))
def test_random_gemv(i):
    S, hc, n, m, B, xdtype = gemv_case(i)
    P = S * (2 if hc else 1)
    log(f"random gemv #{i}: S={S} conj={hc} n={n} m={m} B={B} {DTYPES[xdtype]}")
    codes = synth.random_codes((P, n, m), 7100 + i)
    scales = synth.random_scales(P, 7200 + i)
    layer = layer_from_codes(codes, scales, S, hc)
    xr_d, xi_d, xr, xi = activations(xdtype, B, m, 7300 + i)
    want_acc = xdtype == F.FAIRY_I8
    yr, yi, acc = run_gemv(layer, xr_d, xi_d, xdtype, B, want_acc=want_acc)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr, xi)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
    if want_acc:
        assert np.array_equal(acc.astype(np.int64),
                              oracle.cgemv_acc_i64(codes, xr.astype(np.int8), xi.astype(np.int8)))


def gemm_case(i):
    g = synth.rng(8000 + i)
    S = int(g.integers(1, 5))
    hc = bool(g.integers(0, 2))
    n = int(g.integers(1, 301))
    m = 16 * int(g.integers(1, 129))
    M = int(g.integers(1, 201))
    xdtype = int(g.choice([F.FAIRY_BF16, F.FAIRY_I8]))
    algo = int(g.choice([F.FAIRY_ALGO_AUTO, F.FAIRY_ALGO_VALU, F.FAIRY_ALGO_MFMA]))
    ws = bool(g.integers(0, 2))
    return S, hc, n, m, M, xdtype, algo, ws


@pytest.mark.parametrize("i", range(40))
def test_random_gemm(i):
    S, hc, n, m, M, xdtype, algo, ws = gemm_case(i)
    P = S * (2 if hc else 1)
    log(f"random gemm #{i}: S={S} conj={hc} n={n} m={m} M={M} {DTYPES[xdtype]} algo={algo} workspace={ws}")
    codes = synth.random_codes((P, n, m), 8100 + i)
    scales = synth.random_scales(P, 8200 + i)
    layer = layer_from_codes(codes, scales, S, hc)
    xr_d, xi_d, xr, xi = activations(xdtype, M, m, 8300 + i)
    yr, yi, _ = run_gemv(layer, xr_d, xi_d, xdtype, M, gemm=True, algo=algo, workspace=ws)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr, xi)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


def attention_case(i):
    g = synth.rng(9000 + i)
    h = int(g.integers(1, 4))
    causal = int(g.integers(0, 2))
    sq = int(g.integers(1, 301))
    sk = int(g.integers(sq if causal else 1, 401))
    d = int(g.choice([32, 64, 128]))
    scale = float(g.uniform(-2.0, 2.0)) / np.sqrt(2 * d)
    return h, sq, sk, d, causal, scale


@pytest.mark.parametrize("i", range(30))
def test_random_attention(i):
    h, sq, sk, d, causal, scale = attention_case(i)
    log(f"random attention #{i}: h={h} sq={sq} sk={sk} d={d} causal={causal} scale={scale:.4f}")
    t = torch()
    bits, vals = [], []
    for j, rows in enumerate([sq, sq, sk, sk, sk, sk]):
        b = synth.bf16_bits(synth.gaussian((h, rows, d), 1.0, 9100 + 10 * i + j))
        bits.append(dev(b))
        vals.append(synth.bf16_to_f32(b))
    o_re = t.empty((h, sq, d), dtype=t.float32, device="cuda")
    o_im = t.empty_like(o_re)
    F.fairy_cattention(*bits, F.FAIRY_BF16, h, sq, sk, d, scale, causal, o_re, o_im)
    t.cuda.synchronize()
    w_re, w_im = oracle.cattention(*vals, scale, bool(causal))
    err = rel_l2(host(o_re) + 1j * host(o_im), w_re + 1j * w_im)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
