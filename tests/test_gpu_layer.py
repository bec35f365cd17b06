"""GPU parity of the whole-layer conversion and of the serialised layer.

fairy_quantize_real / fairy_quantize_complex must equal, bit for bit, the
oracle's own steps in the pages' order (widely-linear split rounded to fp32,
PhaseQuant of U and of W with S residual stages, TILED64 packing); a layer
written with fairy_layer_save and read back with fairy_layer_load must be
the same layer (same words, same scales, same GEMV output bits).
"""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import GpuLayer, dev, host, log, run_gemv, torch

pytestmark = pytest.mark.gpu


def quantize_real_gpu(R, n, m, S):
    t = torch()
    P = 2 * S
    packed = t.empty(F.fairy_packed_words(n, m, P, F.FAIRY_LAYOUT_TILED64), dtype=t.int32, device="cuda")
    scales = t.empty((P, 2), dtype=t.float32, device="cuda")
    wsb = F.fairy_quantize_workspace_bytes(n, m, S, 1)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    F.fairy_quantize_real(dev(R), n, m, S, packed, scales, ws, wsb)
    return GpuLayer(n, m, S, True, packed, scales)


def oracle_real(R, n, m, S):
    ure, uim, wre, wim = oracle.real_to_complex(R, n, m, f32=True)
    cu, su, _, _ = oracle.phasequant(ure, uim, S, want_resid=False)
    cw, sw, _, _ = oracle.phasequant(wre, wim, S, want_resid=False)
    codes = np.concatenate([cu, cw])
    return oracle.pack(codes, F.FAIRY_LAYOUT_TILED64), np.concatenate([su, sw]), codes


@pytest.mark.parametrize("n,m,S,seed", [(37, 80, 3, 1), (64, 2048, 1, 2), (2048, 2048, 2, 200)])
def test_quantize_real_bit_exact(n, m, S, seed):
    log(f"quantize_real n={n} m={m} S={S}")
    R = synth.real_layer(2 * n, 2 * m, seed)
    L = quantize_real_gpu(R, n, m, S)
    torch().cuda.synchronize()
    words, scales, _ = oracle_real(R, n, m, S)
    assert np.array_equal(host(L.packed).view(np.uint32), words)
    assert np.array_equal(host(L.scales).view(np.uint32), scales.view(np.uint32))


def test_quantize_real_edge_values():
    """U and W are formed inside the PhaseQuant stages: the split's single
    rounding must hold where an fp32 sum would not give it directly (zero and
    cancelling sums, subnormal halves, halves at the bottom of the normal
    range, sums that overflow fp32) and beside ordinary values in one vector."""
    n, m, S = 64, 256, 2
    R = synth.real_layer(2 * n, 2 * m, 7)
    tiny = np.float32(np.ldexp(1.5, -126))      # R11 + 0 = 1.5 * 2^-126: its half is subnormal
    sub = np.float32(np.ldexp(3.0, -149))       # subnormal input
    low = np.float32(np.ldexp(1.0, -125))       # half exactly 2^-126, the smallest normal
    big = np.float32(3.0e38)                    # big + big overflows fp32, its half does not
    def put(i, j, r11, r12, r21, r22):
        R[i, j], R[i, m + j], R[n + i, j], R[n + i, m + j] = r11, r12, r21, r22
    put(0, 0, 0.0, 0.0, 0.0, 0.0)
    put(0, 1, -0.0, 0.0, -0.0, 0.0)
    put(0, 2, 0.5, 0.25, 0.25, -0.5)            # R11 + R22 = 0, R21 - R12 = 0
    put(1, 4, tiny, 0.0, sub, 0.0)
    put(1, 5, low, -low, low, 0.0)
    put(2, 8, big, big, -big, big)              # Re U, Im W, Re W, Im U from +-big pairs
    put(2, 9, -big, big, big, -big)
    put(3, 12, big, -sub, tiny, -big)
    put(5, 17, sub, sub, -sub, sub)
    log(f"quantize_real edge values n={n} m={m} S={S}")
    L = quantize_real_gpu(R, n, m, S)
    torch().cuda.synchronize()
    words, scales, _ = oracle_real(R, n, m, S)
    assert np.array_equal(host(L.packed).view(np.uint32), words)
    assert np.array_equal(host(L.scales).view(np.uint32), scales.view(np.uint32))


def test_quantize_real_unaligned_input():
    """R 4-byte aligned but not 16: the stages read it one element at a time."""
    n, m, S = 48, 160, 2
    R = synth.real_layer(2 * n, 2 * m, 11)
    t = torch()
    buf = t.zeros(R.size + 4, dtype=t.float32, device="cuda")
    view = buf[1:1 + R.size]
    assert view.data_ptr() % 16 == 4
    view.copy_(dev(R.reshape(-1)))
    P = 2 * S
    packed = t.empty(F.fairy_packed_words(n, m, P, F.FAIRY_LAYOUT_TILED64), dtype=t.int32, device="cuda")
    scales = t.empty((P, 2), dtype=t.float32, device="cuda")
    wsb = F.fairy_quantize_workspace_bytes(n, m, S, 1)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    log(f"quantize_real unaligned n={n} m={m} S={S}")
    F.fairy_quantize_real(view, n, m, S, packed, scales, ws, wsb)
    t.cuda.synchronize()
    words, sc, _ = oracle_real(R, n, m, S)
    assert np.array_equal(host(packed).view(np.uint32), words)
    assert np.array_equal(host(scales).view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("case", range(6))
def test_quantize_real_random_shapes(case):
    g = np.random.default_rng(900 + case)
    n = int(g.integers(1, 200))
    m = 16 * int(g.integers(1, 40))
    S = int(g.integers(1, 4))
    log(f"quantize_real random case={case} n={n} m={m} S={S}")
    R = synth.real_layer(2 * n, 2 * m, 950 + case)
    L = quantize_real_gpu(R, n, m, S)
    torch().cuda.synchronize()
    words, scales, _ = oracle_real(R, n, m, S)
    assert np.array_equal(host(L.packed).view(np.uint32), words)
    assert np.array_equal(host(L.scales).view(np.uint32), scales.view(np.uint32))


@pytest.mark.parametrize("n,m,S,sigma,seed", [(130, 256, 2, 1.0, 3), (2048, 2048, 2, 0.02 / np.sqrt(2), 500)])
def test_quantize_complex_bit_exact(n, m, S, sigma, seed):
    log(f"quantize_complex n={n} m={m} S={S}")
    t = torch()
    re, im = synth.complex_gaussian((n, m), sigma, seed)
    packed = t.empty(F.fairy_packed_words(n, m, S, F.FAIRY_LAYOUT_TILED64), dtype=t.int32, device="cuda")
    scales = t.empty((S, 2), dtype=t.float32, device="cuda")
    wsb = F.fairy_quantize_workspace_bytes(n, m, S, 0)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    F.fairy_quantize_complex(dev(re), dev(im), n, m, S, packed, scales, ws, wsb)
    t.cuda.synchronize()
    codes, sc, _, _ = oracle.phasequant(re, im, S, want_resid=False)
    assert np.array_equal(host(packed).view(np.uint32), oracle.pack(codes, F.FAIRY_LAYOUT_TILED64))
    assert np.array_equal(host(scales).view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("n,m,S", [(37, 80, 2), (300, 512, 3)])
def test_save_load_round_trip(n, m, S):
    log(f"save/load n={n} m={m} S={S}")
    t = torch()
    R = synth.real_layer(2 * n, 2 * m, 7 + n)
    L = quantize_real_gpu(R, n, m, S)
    buf = bytearray(F.fairy_layer_file_bytes(n, m, S, 1))
    F.fairy_layer_save(L.desc, buf)
    info = F.fairy_layer_read_info(buf)
    assert (info.n, info.m, info.stages, info.has_conj, info.planes) == (n, m, S, 1, 2 * S)
    # the header fields sit where include/fairy.h puts them
    assert bytes(buf[:8]) == b"FAIRYQL1"
    assert np.frombuffer(bytes(buf[64:64 + 16 * S]), np.float32).tobytes() == host(L.scales).tobytes()
    assert bytes(buf[info.header_bytes:]) == host(L.packed).tobytes()
    packed2 = t.empty_like(L.packed)
    scales2 = t.empty_like(L.scales)
    F.fairy_layer_load(bytes(buf), packed2, scales2)
    assert t.equal(packed2, L.packed) and t.equal(scales2, L.scales)
    L2 = GpuLayer(n, m, S, True, packed2, scales2)
    rb, ib = synth.bf16_gaussian((3, m), 11)
    y1 = run_gemv(L, dev(rb), dev(ib), F.FAIRY_BF16, 3)
    y2 = run_gemv(L2, dev(rb), dev(ib), F.FAIRY_BF16, 3)
    assert np.array_equal(y1[0], y2[0]) and np.array_equal(y1[1], y2[1])
