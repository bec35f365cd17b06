"""Every entry point captured in a HIP graph: three replays, each after eager
work on the same buffers, must reproduce the eager result bit for bit (the
calls launch only kernels: no memset or copy nodes, no allocation)."""
import numpy as np
import pytest

from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, layer_from_codes, log, torch

pytestmark = pytest.mark.gpu


def replay_check(call, outputs, clobber):
    """Run `call` eagerly, capture it, then three times: clobber the outputs
    with eager work, replay, compare with the eager result."""
    t = torch()
    call()
    t.cuda.synchronize()
    want = [host(o).copy() for o in outputs]
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            call()
    t.cuda.synchronize()
    for rep in range(3):
        clobber()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert np.array_equal(host(o), w), f"replay {rep} differs"


def test_graph_phasequant_and_pack():
    t = torch()
    n, m, S = 300, 512, 2
    re, im = synth.complex_gaussian((n, m), 0.02, 61)
    w_re, w_im = dev(re), dev(im)
    count = n * m
    codes = t.empty(S * count, dtype=t.uint8, device="cuda")
    scales = t.empty(2 * S, dtype=t.float32, device="cuda")
    rr = t.empty(count, dtype=t.float32, device="cuda")
    ri = t.empty(count, dtype=t.float32, device="cuda")
    wsb = F.fairy_phasequant_workspace_bytes(count, S)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    packed = t.empty(F.fairy_packed_words(n, m, S, F.FAIRY_LAYOUT_TILED64), dtype=t.int32, device="cuda")

    def call():
        F.fairy_phasequant(w_re, w_im, count, S, codes, scales, rr, ri, ws, wsb)
        F.fairy_pack(codes, S, n, m, F.FAIRY_LAYOUT_TILED64, packed)

    def clobber():
        for b in (codes, scales, rr, ri, packed, ws):
            b.fill_(7)   # the workspace too: the call must clear what it accumulates into
    log("graph: phasequant + pack")
    replay_check(call, [codes, scales, rr, ri, packed], clobber)


def test_graph_quantize_real():
    """The one-call real-layer conversion (U and W formed inside the
    PhaseQuant stages, two matrices per launch) under replay."""
    t = torch()
    n, m, S = 96, 320, 2
    R = dev(synth.real_layer(2 * n, 2 * m, 65))
    P = 2 * S
    packed = t.empty(F.fairy_packed_words(n, m, P, F.FAIRY_LAYOUT_TILED64), dtype=t.int32, device="cuda")
    scales = t.empty((P, 2), dtype=t.float32, device="cuda")
    wsb = F.fairy_quantize_workspace_bytes(n, m, S, 1)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")

    def clobber():
        for b in (packed, scales, ws):
            b.fill_(7)
    log("graph: quantize_real")
    replay_check(lambda: F.fairy_quantize_real(R, n, m, S, packed, scales, ws, wsb), [packed, scales], clobber)


@pytest.mark.parametrize("xdtype", [F.FAIRY_BF16, F.FAIRY_I8])
def test_graph_gemv(xdtype):
    t = torch()
    n, m, B = 200, 1024, 4
    codes = synth.random_codes((4, n, m), 62)
    layer = layer_from_codes(codes, synth.random_scales(4, 63), 2, True)
    if xdtype == F.FAIRY_BF16:
        xr, xi = (dev(a) for a in synth.bf16_gaussian((B, m), 64))
    else:
        xr, xi = (dev(a) for a in synth.int8_uniform((B, m), 64))
    yr = t.empty((B, n), dtype=t.float32, device="cuda")
    yi = t.empty_like(yr)
    acc = t.empty((4, 4, B, n), dtype=t.int32, device="cuda") if xdtype == F.FAIRY_I8 else None
    outs = [yr, yi] + ([acc] if acc is not None else [])
    log(f"graph: cgemv dtype={xdtype}")
    replay_check(lambda: F.fairy_cgemv(layer.desc, xr, xi, xdtype, B, m, yr, yi, n, acc), outs,
                 lambda: [o.fill_(3) for o in outs])


@pytest.mark.parametrize("M,workspace", [(16, True), (16, False), (200, False)])
def test_graph_gemm_mfma(M, workspace):
    """The matrix-core GEMM, unsplit and split along K (two kernels)."""
    t = torch()
    n, m = 256, 2048
    codes = synth.random_codes((4, n, m), 65)
    layer = layer_from_codes(codes, synth.random_scales(4, 66), 2, True)
    xr, xi = (dev(a) for a in synth.bf16_gaussian((M, m), 67))
    yr = t.empty((M, n), dtype=t.float32, device="cuda")
    yi = t.empty_like(yr)
    wsb = F.fairy_cgemm_workspace_bytes(layer.desc, M, F.FAIRY_BF16, F.FAIRY_ALGO_MFMA) if workspace else 0
    if workspace:
        assert wsb > 0
    ws = t.empty((max(wsb, 16),), dtype=t.uint8, device="cuda") if workspace else None
    log(f"graph: cgemm MFMA M={M} workspace={workspace}")
    replay_check(lambda: F.fairy_cgemm(layer.desc, xr, xi, F.FAIRY_BF16, M, m, yr, yi, n, None, F.FAIRY_ALGO_MFMA,
                                       ws, wsb),
                 [yr, yi], lambda: [yr.fill_(5), yi.fill_(5)] + ([ws.fill_(9)] if ws is not None else []))


def test_graph_gemv_lut():
    t = torch()
    n, m = 1000, 2048
    codes = synth.random_codes((4, n, m), 68)
    layer = layer_from_codes(codes, synth.random_scales(4, 69), 2, True)
    xr, xi = (dev(a) for a in synth.bf16_gaussian((1, m), 70))
    yr = t.empty((1, n), dtype=t.float32, device="cuda")
    yi = t.empty_like(yr)
    wsb = F.fairy_cgemv_lut_workspace_bytes(layer.desc)
    ws = t.empty((max(wsb, 16),), dtype=t.uint8, device="cuda")
    log("graph: cgemv_lut")
    replay_check(lambda: F.fairy_cgemv_lut(layer.desc, xr, xi, F.FAIRY_BF16, yr, yi, ws, wsb), [yr, yi],
                 lambda: [yr.fill_(1), yi.fill_(1), ws.fill_(2)])


def test_graph_attention():
    t = torch()
    h, sq, sk, d = 2, 150, 300, 64
    bufs = [dev(synth.bf16_bits(synth.gaussian((h, r, d), 1.0, 71 + i))) for i, r in enumerate([sq, sq, sk, sk, sk, sk])]
    o_re = t.empty((h, sq, d), dtype=t.float32, device="cuda")
    o_im = t.empty_like(o_re)
    log("graph: cattention causal")
    replay_check(lambda: F.fairy_cattention(*bufs, F.FAIRY_BF16, h, sq, sk, d, 0.088, 1, o_re, o_im), [o_re, o_im],
                 lambda: [o_re.fill_(4), o_im.fill_(4)])
