"""GPU parity of the complex GEMV / GEMM against the CPU oracle.

Float activations: relative L2 error <= 1e-5 against the fp64 oracle on the
same (bf16- or fp32-valued) inputs.  int8 activations: the int32
accumulators equal the oracle's exact int64 sums.  Codes and scales of the
end-to-end cases are produced on the GPU from the same seeded weights that
the oracle quantises on the CPU.
"""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import (dev, host, layer_from_codes, log, quantize_widely_linear_on_gpu, rel_l2, run_gemv,
                        torch)

pytestmark = pytest.mark.gpu
TOL = 1e-5


def x_bf16(B, m, seed):
    re_b, im_b = synth.bf16_gaussian((B, m), seed)
    return re_b, im_b, synth.bf16_to_f32(re_b), synth.bf16_to_f32(im_b)


def check_float(layer, codes, scales, S, hc, B, xdtype, seed):
    m = layer.m
    if xdtype == F.FAIRY_BF16:
        rb, ib, xr, xi = x_bf16(B, m, seed)
        yr, yi, _ = run_gemv(layer, dev(rb), dev(ib), xdtype, B)
    else:
        xr, xi = synth.complex_gaussian((B, m), 1.0, seed)
        yr, yi, _ = run_gemv(layer, dev(xr), dev(xi), xdtype, B)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr, xi)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
    return yr, yi


# --- the 256x256 single GEMV: one stage, no conjugate branch ----------------------
def test_c1_single_gemv_f32_and_i8():
    log("256x256 S=1 no-conj f32 + i8")
    re, im = synth.complex_gaussian((256, 256), 1.0, 0)
    codes, scales, _, _ = oracle.phasequant(re, im, 1, want_resid=False)
    layer = layer_from_codes(codes, scales, 1, False)
    check_float(layer, codes, scales, 1, False, 1, F.FAIRY_F32, 1)
    xr, xi = synth.int8_uniform((1, 256), 2)
    yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, 1, want_acc=True)
    want = oracle.cgemv_acc_i64(codes, xr, xi)
    assert np.array_equal(acc.astype(np.int64), want)
    wr, wi = oracle.cgemv_dense(codes, scales, 1, False, xr.astype(np.float64), xi.astype(np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


# --- random codes: shapes, tails, plane counts, batch sizes ------------------------
CASES = [
    # (S, has_conj, n, m, B)
    (1, False, 1, 16, 1),
    (1, True, 5, 64, 2),
    (2, True, 37, 80, 3),        # ragged rows and a half-empty column group
    (3, True, 64, 208, 5),
    (2, False, 100, 1024, 8),
    (4, True, 9, 128, 9),        # P = 8
    (8, True, 3, 64, 2),         # P = 16
    (2, True, 130, 2048, 16),
    (2, True, 64, 5504, 4),
    (1, True, 20, 256, 64),
    # one row per wave with lane-fixed planes (P | 64, >= 64 units per row)
    (1, False, 7, 4112, 3),      # P = 1, ragged last group
    (1, True, 33, 2064, 5),      # P = 2
    (4, True, 19, 528, 6),       # P = 8
    (8, True, 5, 272, 2),        # P = 16
    # one row per wave with idle lanes (P does not divide 64: 60 or 63 lanes)
    (3, True, 21, 704, 3),       # P = 6, 11 groups: a second, partial step
    (3, False, 17, 1360, 2),     # P = 3, ragged last group
    (3, True, 40, 2048, 16),     # P = 6, the 2048-column shape
    (3, True, 9, 1024, 64),      # P = 6, batch 64
    (2, True, 9, 1024, 64),      # P = 4, batch 64 in chunks of 4 (int8: the one-row-per-wave kernel)
]


@pytest.mark.parametrize("S,hc,n,m,B", CASES)
@pytest.mark.parametrize("xdtype", [F.FAIRY_BF16, F.FAIRY_F32])
def test_gemv_float_random_codes(S, hc, n, m, B, xdtype):
    log(f"gemv float S={S} conj={hc} n={n} m={m} B={B} dt={xdtype}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 7 * n + m)
    scales = synth.random_scales(P, n + 3 * m)
    layer = layer_from_codes(codes, scales, S, hc)
    check_float(layer, codes, scales, S, hc, B, xdtype, 11 + B)


@pytest.mark.parametrize("S,hc,n,m,B", CASES)
def test_gemv_i8_exact(S, hc, n, m, B):
    log(f"gemv i8 S={S} conj={hc} n={n} m={m} B={B}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 5 * n + m)
    scales = synth.random_scales(P, n + m)
    layer = layer_from_codes(codes, scales, S, hc)
    xr, xi = synth.int8_uniform((B, m), 3 + B)
    yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, B, want_acc=True)
    assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr.astype(np.float64), xi.astype(np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


# the widest layers one staged activation column allows, two batch columns
# (staged one at a time)
@pytest.mark.parametrize("xdtype,m", [(F.FAIRY_BF16, 14528), (F.FAIRY_F32, 7680), (F.FAIRY_I8, 26112)])
def test_gemv_max_m(xdtype, m):
    S, hc, n, B = 2, True, 4, 2
    log(f"gemv max m dt={xdtype} m={m}")
    P = 2 * S
    codes = synth.random_codes((P, n, m), 17 + m)
    scales = synth.random_scales(P, 19 + m)
    layer = layer_from_codes(codes, scales, S, hc)
    if xdtype == F.FAIRY_I8:
        xr, xi = synth.int8_uniform((B, m), 23)
        yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), xdtype, B, want_acc=True)
        assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))
        wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr.astype(np.float64), xi.astype(np.float64))
        assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL
    else:
        check_float(layer, codes, scales, S, hc, B, xdtype, 29)


def test_gemv_extreme_int8_values():
    """All-(+-127) activations and all-equal codes: the largest exact sums."""
    S, n, m = 2, 8, 2048
    for c in range(4):
        codes = np.full((2 * S, n, m), c, np.uint8)
        layer = layer_from_codes(codes, np.ones((2 * S, 2), np.float32), S, True)
        for v in (127, -127):
            xr = np.full((2, m), v, np.int8); xi = np.full((2, m), -v, np.int8)
            _, _, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, 2, want_acc=True)
            assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))


def test_gemv_deterministic():
    codes = synth.random_codes((4, 256, 2048), 1)
    scales = synth.random_scales(4, 2)
    layer = layer_from_codes(codes, scales, 2, True)
    rb, ib, _, _ = x_bf16(4, 2048, 3)
    a = run_gemv(layer, dev(rb), dev(ib), F.FAIRY_BF16, 4)
    b = run_gemv(layer, dev(rb), dev(ib), F.FAIRY_BF16, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_gemv_respects_strides():
    """ldx > m and ldy > n: padding columns/rows are neither read nor written."""
    t = torch()
    S, n, m, B = 1, 40, 64, 3
    codes = synth.random_codes((2, n, m), 4)
    scales = synth.random_scales(2, 5)
    layer = layer_from_codes(codes, scales, S, True)
    xr, xi = synth.complex_gaussian((B, m), 1.0, 6)
    ldx, ldy = 96, 50
    Xr = np.full((B, ldx), np.nan, np.float32); Xr[:, :m] = xr
    Xi = np.full((B, ldx), np.nan, np.float32); Xi[:, :m] = xi
    yr = t.full((B, ldy), 7.0, device="cuda"); yi = t.full((B, ldy), 7.0, device="cuda")
    F.fairy_cgemv(layer.desc, dev(Xr), dev(Xi), F.FAIRY_F32, B, ldx, yr, yi, ldy)
    t.cuda.synchronize()
    yr, yi = host(yr), host(yi)
    assert np.all(yr[:, n:] == 7.0) and np.all(yi[:, n:] == 7.0)
    wr, wi = oracle.cgemv_dense(codes, scales, S, True, xr, xi)
    assert rel_l2(yr[:, :n] + 1j * yi[:, :n], wr + 1j * wi) <= TOL


# --- LLaMA-2-7B-shaped widely-linear layers, quantised on the GPU -------------------
def widely_linear_case(rows, cols, seed, S):
    """Real [rows][cols] sigma=0.02 -> complex U, W [rows/2][cols/2] -> S stages,
    on the GPU; the oracle does the same on the CPU."""
    t = torch()
    n, m = rows // 2, cols // 2
    R = synth.real_layer(rows, cols, seed)
    planes = [t.empty((n, m), dtype=t.float32, device="cuda") for _ in range(4)]
    F.fairy_real_to_complex(dev(R), n, m, *planes)
    layer, gcodes, gscales = quantize_widely_linear_on_gpu(*planes, n, m, S)
    ur, ui, wr, wi = oracle.real_to_complex(R, n, m, f32=True)
    cu, su, _, _ = oracle.phasequant(ur, ui, S, want_resid=False)
    cw, sw, _, _ = oracle.phasequant(wr, wi, S, want_resid=False)
    codes = np.concatenate([cu, cw])
    scales = np.concatenate([su, sw])
    t.cuda.synchronize()
    assert np.array_equal(host(gcodes).reshape(codes.shape), codes)
    assert np.array_equal(host(gscales).reshape(scales.shape).view(np.uint32), scales.view(np.uint32))
    return layer, codes, scales


@pytest.mark.parametrize("B", [1, 4, 16])
def test_llama_attention_shape_s2(B):
    log(f"widely-linear 4096x4096 -> 2048x2048 S=2 B={B}")
    layer, codes, scales = widely_linear_case(4096, 4096, 200, 2)
    check_float(layer, codes, scales, 2, True, B, F.FAIRY_BF16, 201)


@pytest.mark.parametrize("B", [1, 8])
def test_llama_attention_shape_s2_int8(B):
    """The 2048x2048 decode layer with int8 activations: the raw int32
    accumulators of 64 sampled rows equal the oracle's exact sums, and every
    output is within the float bound."""
    log(f"widely-linear 4096x4096 -> 2048x2048 S=2 int8 B={B}")
    layer, codes, scales = widely_linear_case(4096, 4096, 200, 2)
    xr, xi = synth.int8_uniform((B, 2048), 205 + B)
    yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, B, want_acc=True)
    rows = np.sort(synth.rng(206).choice(2048, 64, replace=False))
    want_acc = oracle.cgemv_acc_i64(codes[:, rows], xr, xi)
    assert np.array_equal(acc[:, :, :, rows].astype(np.int64), want_acc)
    wr, wi = oracle.cgemv_dense(codes, scales, 2, True, xr.astype(np.float64), xi.astype(np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


@pytest.mark.parametrize("rows,cols,seed", [(11008, 4096, 300), (4096, 11008, 302)])
@pytest.mark.parametrize("B", [1, 8])
def test_llama_mlp_shapes_s2(rows, cols, seed, B):
    log(f"widely-linear {rows}x{cols} S=2 B={B}")
    layer, codes, scales = widely_linear_case(rows, cols, seed, 2)
    check_float(layer, codes, scales, 2, True, B, F.FAIRY_BF16, seed + 1)


# --- prefill GEMM ----------------------------------------------------------------------
GEMM_CASES = [
    # (S, has_conj, n, m, M)
    (1, False, 16, 64, 1),
    (2, True, 37, 80, 5),          # ragged rows, tokens and column group
    (3, True, 300, 256, 77),
    (1, False, 64, 2048, 64),
    (2, True, 257, 512, 33),
    (4, True, 40, 128, 40),        # P = 8
    (1, True, 130, 320, 65),       # P = 2
    (3, False, 50, 192, 70),       # P = 3: a 2-plane pass, then a 1-plane pass adding into y
    (7, False, 33, 64, 129),       # P = 7: 4 + 2 + 1 planes, three token blocks
    (2, True, 70, 192, 24),        # 32-token blocks (17..32 tokens), ragged
    (3, True, 100, 128, 17),       # 32-token blocks, P = 6: a 4-plane then a 2-plane pass
    (7, False, 33, 64, 16),        # 16-token blocks, P = 7 in three passes
]


@pytest.mark.parametrize("S,hc,n,m,M", GEMM_CASES)
@pytest.mark.parametrize("algo", [F.FAIRY_ALGO_MFMA, F.FAIRY_ALGO_VALU])
def test_gemm_bf16_full(S, hc, n, m, M, algo):
    log(f"gemm bf16 algo={algo} S={S} conj={hc} n={n} m={m} M={M}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 3 * n + m + M)
    scales = synth.random_scales(P, n + M)
    layer = layer_from_codes(codes, scales, S, hc)
    rb, ib, xr, xi = x_bf16(M, m, 17 + M)
    yr, yi, _ = run_gemv(layer, dev(rb), dev(ib), F.FAIRY_BF16, M, gemm=True, algo=algo)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr, xi)
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


@pytest.mark.parametrize("S,hc,n,m,M", GEMM_CASES)
@pytest.mark.parametrize("algo", [F.FAIRY_ALGO_MFMA, F.FAIRY_ALGO_VALU])
def test_gemm_i8_exact(S, hc, n, m, M, algo):
    log(f"gemm i8 algo={algo} S={S} conj={hc} n={n} m={m} M={M}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 2 * n + m + M)
    scales = synth.random_scales(P, n + 2 * M)
    layer = layer_from_codes(codes, scales, S, hc)
    xr, xi = synth.int8_uniform((M, m), 5 + M)
    yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, M, want_acc=True, gemm=True, algo=algo)
    assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr.astype(np.float64), xi.astype(np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


# K split of the matrix-core GEMM at token counts that leave CUs idle
SPLIT_CASES = [
    # (S, has_conj, n, m, M, xdtype)
    (2, True, 2048, 2048, 16, F.FAIRY_BF16),    # the decode-batch case: 8 splits of 2 chunks
    (2, True, 2048, 2048, 64, F.FAIRY_I8),      # 8 splits of 1 chunk
    (1, False, 200, 1088, 5, F.FAIRY_BF16),     # P = 1, ragged rows and a half-full last chunk
    (1, True, 130, 2064, 33, F.FAIRY_I8),       # P = 2, 33 groups: a one-group last chunk
    (2, True, 5504, 2048, 8, F.FAIRY_BF16),     # 86 row blocks: 3 splits of 6, 6, 4 chunks
    (2, True, 300, 4096, 150, F.FAIRY_BF16),    # 3 token blocks, ragged tokens
    (2, True, 2048, 2048, 32, F.FAIRY_BF16),    # 32-token blocks: 8 splits of 2 chunks
    (2, True, 1000, 2048, 20, F.FAIRY_I8),      # 32-token blocks, ragged rows and tokens
]


@pytest.mark.parametrize("S,hc,n,m,M,xdtype", SPLIT_CASES)
def test_gemm_mfma_split_k(S, hc, n, m, M, xdtype):
    log(f"gemm split-K dt={xdtype} S={S} conj={hc} n={n} m={m} M={M}")
    P = S * (2 if hc else 1)
    codes = synth.random_codes((P, n, m), 5 * n + m + M)
    scales = synth.random_scales(P, n + 3 * M)
    layer = layer_from_codes(codes, scales, S, hc)
    assert F.fairy_cgemm_workspace_bytes(layer.desc, M, xdtype, F.FAIRY_ALGO_MFMA) > 0
    if xdtype == F.FAIRY_BF16:
        rb, ib, xr, xi = x_bf16(M, m, 23 + M)
        args = (dev(rb), dev(ib))
    else:
        xr, xi = synth.int8_uniform((M, m), 29 + M)
        args = (dev(xr), dev(xi))
        xr, xi = xr.astype(np.float64), xi.astype(np.float64)
    yr, yi, _ = run_gemv(layer, *args, xdtype, M, gemm=True, algo=F.FAIRY_ALGO_MFMA, workspace=True)
    wr, wi = oracle.cgemv_dense(codes, scales, S, hc, xr, xi)
    err = rel_l2(yr + 1j * yi, wr + 1j * wi)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL
    # the unsplit launch (no workspace) agrees within the same bound
    ur, ui, _ = run_gemv(layer, *args, xdtype, M, gemm=True, algo=F.FAIRY_ALGO_MFMA)
    assert rel_l2(ur + 1j * ui, wr + 1j * wi) <= TOL
    # and the split launch repeats bit for bit
    zr, zi, _ = run_gemv(layer, *args, xdtype, M, gemm=True, algo=F.FAIRY_ALGO_MFMA, workspace=True)
    assert np.array_equal(yr, zr) and np.array_equal(yi, zi)


@pytest.mark.parametrize("xdtype,m", [(F.FAIRY_BF16, 16384), (F.FAIRY_I8, 28672)])
def test_gemm_mfma_beyond_gemv_width(xdtype, m):
    """The matrix-core GEMM streams activations in chunks, so it takes rows
    wider than the GEMV can stage (14528 bf16, 26112 int8 columns)."""
    n, M = 96, 40
    codes = synth.random_codes((2, n, m), 41)
    scales = synth.random_scales(2, 42)
    layer = layer_from_codes(codes, scales, 1, True)
    if xdtype == F.FAIRY_BF16:
        rb, ib, xr, xi = x_bf16(M, m, 43)
        args = (dev(rb), dev(ib))
    else:
        xr, xi = synth.int8_uniform((M, m), 44)
        args = (dev(xr), dev(xi))
    yr, yi, acc = run_gemv(layer, *args, xdtype, M, want_acc=xdtype == F.FAIRY_I8, gemm=True,
                           algo=F.FAIRY_ALGO_MFMA)
    wr, wi = oracle.cgemv_dense(codes, scales, 1, True, np.asarray(xr, np.float64), np.asarray(xi, np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL
    if xdtype == F.FAIRY_I8:
        assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))


def test_gemm_mfma_split_k_with_acc_runs_unsplit():
    """Raw int8 accumulators are exact per plane, so with acc requested the
    call ignores the workspace and runs unsplit."""
    codes = synth.random_codes((4, 256, 2048), 31)
    scales = synth.random_scales(4, 32)
    layer = layer_from_codes(codes, scales, 2, True)
    xr, xi = synth.int8_uniform((16, 2048), 33)
    yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), F.FAIRY_I8, 16, want_acc=True, gemm=True,
                           algo=F.FAIRY_ALGO_MFMA, workspace=True)
    assert np.array_equal(acc.astype(np.int64), oracle.cgemv_acc_i64(codes, xr, xi))
    wr, wi = oracle.cgemv_dense(codes, scales, 2, True, xr.astype(np.float64), xi.astype(np.float64))
    assert rel_l2(yr + 1j * yi, wr + 1j * wi) <= TOL


def test_gemm_mfma_deterministic():
    codes = synth.random_codes((4, 256, 512), 8)
    layer = layer_from_codes(codes, synth.random_scales(4, 9), 2, True)
    rb, ib, _, _ = x_bf16(128, 512, 10)
    a = run_gemv(layer, dev(rb), dev(ib), F.FAIRY_BF16, 128, gemm=True, algo=F.FAIRY_ALGO_MFMA)
    b = run_gemv(layer, dev(rb), dev(ib), F.FAIRY_BF16, 128, gemm=True, algo=F.FAIRY_ALGO_MFMA)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n", [2048, 5504])
@pytest.mark.parametrize("xdtype", [F.FAIRY_BF16, F.FAIRY_I8])
@pytest.mark.parametrize("algo", [F.FAIRY_ALGO_MFMA, F.FAIRY_ALGO_VALU])
def test_prefill_gemm_sampled(n, xdtype, algo):
    """The prefill case at full size: M = 2048 tokens, 2048-column complex
    layers with 2048 or 5504 rows, S = 2 widely-linear; sampled outputs
    (every algorithm: the vector-ALU path against the matrix-core path)."""
    log(f"prefill M=2048 n={n} m=2048 S=2 dt={xdtype} algo={algo}")
    S, m, M = 2, 2048, 2048
    codes = synth.random_codes((2 * S, n, m), 400 + n)
    scales = synth.random_scales(2 * S, 401)
    layer = layer_from_codes(codes, scales, S, True)
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((M, m), 402)
        xr, xi = synth.bf16_to_f32(rb), synth.bf16_to_f32(ib)
        yr, yi, _ = run_gemv(layer, dev(rb), dev(ib), xdtype, M, gemm=True, algo=algo)
    else:
        xr, xi = synth.int8_uniform((M, m), 403)
        yr, yi, acc = run_gemv(layer, dev(xr), dev(xi), xdtype, M, want_acc=True, gemm=True, algo=algo)
    g = synth.rng(404)
    rows = np.sort(g.choice(n, 48, replace=False))
    toks = np.sort(g.choice(M, 48, replace=False))
    wr, wi = oracle.cgemv_dense(codes[:, rows], scales, S, True, xr[toks].astype(np.float64),
                                xi[toks].astype(np.float64))
    got = yr[np.ix_(toks, rows)] + 1j * yi[np.ix_(toks, rows)]
    assert rel_l2(got, wr + 1j * wi) <= TOL
    if xdtype == F.FAIRY_I8:
        want_acc = oracle.cgemv_acc_i64(codes[:, rows], xr[toks], xi[toks])
        assert np.array_equal(acc[:, :, toks][:, :, :, rows].astype(np.int64), want_acc)


@pytest.mark.parametrize("xdtype", [F.FAIRY_BF16, F.FAIRY_I8])
def test_prefill_gemm_full_output(xdtype):
    """The prefill case at full size compared on every output: M = 2048
    tokens through the 2048x2048 S = 2 widely-linear layer, on the matrix
    cores and on the vector ALUs.  int8: every raw accumulator exact; floats
    within the bound.  The oracle runs on all host cores (each output is
    still one ordered sum)."""
    S, n, m, M = 2, 2048, 2048, 2048
    log(f"prefill full output M={M} n={n} m={m} S={S} dt={xdtype}")
    codes = synth.random_codes((2 * S, n, m), 410)
    scales = synth.random_scales(2 * S, 411)
    layer = layer_from_codes(codes, scales, S, True)
    oracle.set_threads(0)
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((M, m), 412)
        xr, xi = synth.bf16_to_f32(rb), synth.bf16_to_f32(ib)
        args = (dev(rb), dev(ib))
    else:
        xr, xi = synth.int8_uniform((M, m), 413)
        args = (dev(xr), dev(xi))
    wr, wi = oracle.cgemv_dense(codes, scales, S, True, xr.astype(np.float64), xi.astype(np.float64))
    want_acc = oracle.cgemv_acc_i64(codes, xr, xi) if xdtype == F.FAIRY_I8 else None
    for algo in (F.FAIRY_ALGO_MFMA, F.FAIRY_ALGO_VALU):
        yr, yi, acc = run_gemv(layer, *args, xdtype, M, want_acc=xdtype == F.FAIRY_I8, gemm=True, algo=algo)
        err = rel_l2(yr + 1j * yi, wr + 1j * wi)
        log(f"  algo={algo} rel_l2={err:.3e}")
        assert err <= TOL
        if want_acc is not None:
            assert np.array_equal(acc.astype(np.int64), want_acc)
        del acc
