"""GPU parity of the grouped decode GEMV (fairy_cgemv_group): several layers
that read the same activations in one launch.  Every layer's output is
within the float bound of the fp64 oracle and equal, bit for bit, to what
fairy_cgemv gives for that layer alone (the same kernel body, the same
summation order)."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, layer_from_codes, log, quantize_widely_linear_on_gpu, rel_l2, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5


def activations(xdtype, B, m, seed):
    """(device re, device im, float64 re, float64 im)"""
    if xdtype == F.FAIRY_BF16:
        rb, ib = synth.bf16_gaussian((B, m), seed)
        return dev(rb), dev(ib), synth.bf16_to_f32(rb).astype(np.float64), synth.bf16_to_f32(ib).astype(np.float64)
    if xdtype == F.FAIRY_F32:
        xr, xi = synth.complex_gaussian((B, m), 1.0, seed)
        return dev(xr), dev(xi), xr.astype(np.float64), xi.astype(np.float64)
    xr, xi = synth.int8_uniform((B, m), seed)
    return dev(xr), dev(xi), xr.astype(np.float64), xi.astype(np.float64)


def run_group(layers, xr, xi, xdtype, B, m, ldy_pad=0):
    t = torch()
    ys = [(t.full((B, L.n + ldy_pad), 7.0, dtype=t.float32, device="cuda"),
           t.full((B, L.n + ldy_pad), 7.0, dtype=t.float32, device="cuda")) for L in layers]
    F.fairy_cgemv_group([L.desc for L in layers], xr, xi, xdtype, B, m, [y[0] for y in ys], [y[1] for y in ys],
                        [L.n + ldy_pad for L in layers])
    t.cuda.synchronize()
    return [(host(a), host(b)) for a, b in ys]


def run_single(L, xr, xi, xdtype, B, m):
    t = torch()
    yr = t.empty((B, L.n), dtype=t.float32, device="cuda")
    yi = t.empty((B, L.n), dtype=t.float32, device="cuda")
    F.fairy_cgemv(L.desc, xr, xi, xdtype, B, m, yr, yi, L.n)
    t.cuda.synchronize()
    return host(yr), host(yi)


CASES = [
    # (S, has_conj, row counts, m, B, dtype)
    (2, True, (256, 256, 256), 2048, 1, F.FAIRY_BF16),          # q, k, v
    (2, True, (1000, 17, 64, 200), 2048, 3, F.FAIRY_BF16),     # ragged rows: blocks split unevenly
    (2, True, (300, 129), 5504, 8, F.FAIRY_BF16),               # gate, up width, ragged last group
    (1, False, (100, 333), 4096, 16, F.FAIRY_BF16),
    (3, True, (77, 130), 1024, 5, F.FAIRY_BF16),                # P = 6: 60 of 64 lanes
    (2, True, (128, 96, 40), 1024, 4, F.FAIRY_F32),
    (2, True, (256, 70, 33), 2048, 1, F.FAIRY_I8),              # grouped int8 kernel (P = 4)
    (2, True, (64, 65), 2048, 64, F.FAIRY_I8),
    (3, True, (50, 60), 1024, 2, F.FAIRY_I8),                   # P = 6 int8: layer by layer
    (1, False, (40, 41, 42), 256, 2, F.FAIRY_BF16),             # rows of 4 units: layer by layer
    (8, True, (33,) * 8, 1024, 1, F.FAIRY_BF16),                # eight layers, P = 16
]


@pytest.mark.parametrize("S,hc,rows,m,B,xdtype", CASES)
def test_group_matches_oracle_and_single(S, hc, rows, m, B, xdtype):
    log(f"group S={S} conj={hc} rows={rows} m={m} B={B} dt={xdtype}")
    P = S * (2 if hc else 1)
    layers, codes, scales = [], [], []
    for i, n in enumerate(rows):
        c = synth.random_codes((P, n, m), 700 + 13 * i + n + m)
        sc = synth.random_scales(P, 701 + i)
        codes.append(c)
        scales.append(sc)
        layers.append(layer_from_codes(c, sc, S, hc))
    xr, xi, fr, fi = activations(xdtype, B, m, 702 + B)
    got = run_group(layers, xr, xi, xdtype, B, m)
    for i, L in enumerate(layers):
        wr, wi = oracle.cgemv_dense(codes[i], scales[i], S, hc, fr, fi)
        err = rel_l2(got[i][0] + 1j * got[i][1], wr + 1j * wi)
        log(f"  layer {i} rows={L.n} rel_l2={err:.3e}")
        assert err <= TOL
        sr, si = run_single(L, xr, xi, xdtype, B, m)
        assert np.array_equal(got[i][0], sr) and np.array_equal(got[i][1], si)


def test_group_attention_projections_end_to_end():
    """q, k and v of the LLaMA-2-7B attention layer shape, each converted
    from its own seeded real 4096x4096 weights and quantised (S = 2) on the
    GPU, applied to one bf16 activation vector in one call; padded output
    rows (ldy > n) are left untouched."""
    t = torch()
    S, n, m = 2, 2048, 2048
    layers, ref = [], []
    for i in range(3):
        R = synth.real_layer(2 * n, 2 * m, 210 + i)
        planes = [t.empty((n, m), dtype=t.float32, device="cuda") for _ in range(4)]
        F.fairy_real_to_complex(dev(R), n, m, *planes)
        L, cd, sc = quantize_widely_linear_on_gpu(*planes, n, m, S)
        layers.append(L)
        ref.append((host(cd).reshape(2 * S, n, m), host(sc).reshape(2 * S, 2)))
    xr, xi, fr, fi = activations(F.FAIRY_BF16, 1, m, 213)
    got = run_group(layers, xr, xi, F.FAIRY_BF16, 1, m, ldy_pad=5)
    for i in range(3):
        wr, wi = oracle.cgemv_dense(ref[i][0], ref[i][1], S, True, fr, fi)
        assert rel_l2(got[i][0][:, :n] + 1j * got[i][1][:, :n], wr + 1j * wi) <= TOL
        assert np.all(got[i][0][:, n:] == 7.0) and np.all(got[i][1][:, n:] == 7.0)
        sr, si = run_single(layers[i], xr, xi, F.FAIRY_BF16, 1, m)
        assert np.array_equal(got[i][0][:, :n], sr) and np.array_equal(got[i][1][:, :n], si)


def test_group_repeatable():
    codes = synth.random_codes((4, 512, 2048), 720)
    L = layer_from_codes(codes, synth.random_scales(4, 721), 2, True)
    xr, xi, _, _ = activations(F.FAIRY_BF16, 2, 2048, 722)
    a = run_group([L, L], xr, xi, F.FAIRY_BF16, 2, 2048)
    b = run_group([L, L], xr, xi, F.FAIRY_BF16, 2, 2048)
    for (ar, ai), (br, bi) in zip(a, b):
        assert np.array_equal(ar, br) and np.array_equal(ai, bi)
    assert np.array_equal(a[0][0], a[1][0]) and np.array_equal(a[0][1], a[1][1])
