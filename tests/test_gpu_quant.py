"""GPU parity of the offline steps (conversion, PhaseQuant, packing) against
the CPU oracle: bit-exact on every code, scale, residual, converted weight
and packed word."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, log, pack_on_gpu, phasequant_on_gpu, torch

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("n,m,seed", [(1, 1, 1), (3, 5, 2), (64, 48, 3), (2048, 2048, 200),
                                      (5504, 2048, 300), (2048, 5504, 302)])
def test_real_to_complex_bit_exact(n, m, seed):
    log(f"real_to_complex n={n} m={m}")
    R = synth.real_layer(2 * n, 2 * m, seed)
    want = oracle.real_to_complex(R, n, m, f32=True)
    t = torch()
    outs = [t.empty((n, m), dtype=t.float32, device="cuda") for _ in range(4)]
    F.fairy_real_to_complex(dev(R), n, m, *outs)
    t.cuda.synchronize()
    for o, w in zip(outs, want):
        assert np.array_equal(bits(host(o)), bits(w))


def _check_pq(re, im, stages):
    count = re.size
    log(f"phasequant count={count} stages={stages}")
    codes_w, scales_w, rr_w, ri_w = oracle.phasequant(re.ravel(), im.ravel(), stages)
    codes, scales, rr, ri = phasequant_on_gpu(dev(re.ravel()), dev(im.ravel()), count, stages)
    torch().cuda.synchronize()
    assert np.array_equal(bits(host(scales).reshape(stages, 2)), bits(scales_w))
    assert np.array_equal(host(codes).reshape(stages, count), codes_w.reshape(stages, count))
    assert np.array_equal(bits(host(rr)), bits(rr_w)) and np.array_equal(bits(host(ri)), bits(ri_w))


@pytest.mark.parametrize("shape,sigma,seed,stages", [
    ((256, 256), 1.0, 0, 1),          # the 256x256 single-GEMV case
    ((1,), 1.0, 5, 1), ((7,), 1.0, 6, 3), ((1000, 3), 0.5, 7, 2),
    ((2048, 2048), 0.02 / np.sqrt(2), 9, 2),
    ((300, 77), 1.0, 10, 8),
    ((2049, 3), 0.3, 11, 3),          # odd count: the one-element-per-thread path, many blocks
])
def test_phasequant_bit_exact(shape, sigma, seed, stages):
    re, im = synth.complex_gaussian(shape, sigma, seed)
    _check_pq(re, im, stages)


def test_phasequant_edge_values():
    g = synth.rng(44)
    k = 4096
    re = g.standard_normal(k).astype(np.float32)
    im = g.standard_normal(k).astype(np.float32)
    im[:512] = re[:512] * np.where(g.random(512) < 0.5, -1, 1).astype(np.float32)   # exact ties
    re[512:600] = 0.0; im[512:600] = 0.0                                            # zeros
    re[600:650] = -0.0
    e = g.integers(-149, -120, 400).astype(np.float64)                              # subnormal / tiny
    re[700:1100] = (g.random(400) * np.exp2(e)).astype(np.float32)
    im[700:1100] = (g.random(400) * np.exp2(e - 1)).astype(np.float32)
    re[1200:1300] = 3e38; im[1300:1400] = -3e38                                     # huge
    _check_pq(re, im, 3)


@pytest.mark.parametrize("count", [3000, 4097])
def test_phasequant_all_zero(count):
    """A zero matrix (both signs of zero): every code 0, s_re the mean of
    zeros and s_im over an empty set, both 0, and the residuals keep each
    zero's sign (x - 0 is x)."""
    g = np.random.default_rng(count)
    re = np.where(g.random(count) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    im = np.where(g.random(count) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    _check_pq(re, im, 3)


def test_phasequant_all_one_axis():
    """Every code on the real axis: s_im's set is empty, so s_im = 0."""
    re = synth.gaussian(1000, 1.0, 3)
    im = np.zeros(1000, np.float32)
    _check_pq(re, im, 2)


@pytest.mark.parametrize("layout", [F.FAIRY_LAYOUT_ROW16, F.FAIRY_LAYOUT_TILED64])
@pytest.mark.parametrize("planes,rows,m", [(1, 1, 16), (1, 256, 256), (4, 37, 80), (3, 129, 2096), (6, 5, 5504),
                                           (4, 2048, 2048)])
def test_pack_unpack_bit_exact(layout, planes, rows, m):
    log(f"pack layout={layout} planes={planes} rows={rows} m={m}")
    c = synth.random_codes((planes, rows, m), 1000 + rows)
    want = oracle.pack(c, layout)
    packed = pack_on_gpu(dev(c), planes, rows, m, layout)
    t = torch()
    back = t.empty(planes * rows * m, dtype=t.uint8, device="cuda")
    F.fairy_unpack(packed, planes, rows, m, layout, back)
    t.cuda.synchronize()
    assert np.array_equal(host(packed, np.uint32), want)
    assert np.array_equal(host(back).reshape(planes, rows, m), c)


def test_pack_ignores_high_bits():
    c = synth.random_codes((1, 4, 64), 5)
    noisy = (c | (synth.random_codes((1, 4, 64), 6) << 2)).astype(np.uint8)
    packed = pack_on_gpu(dev(noisy), 1, 4, 64)
    torch().cuda.synchronize()
    assert np.array_equal(host(packed, np.uint32), oracle.pack(c, oracle.TILED64))


def test_phasequant_scale_rounding_fixtures():
    """The hand-worked mean-rounding cases (ties to even, subnormal means) as
    real-axis weights: s_re must be the fixture value, s_im 0."""
    from tests._golden import hex_to_f32, rows
    for line in rows("abs_mean_rounding.txt"):
        want, vals = line.split(";")
        re = np.array([hex_to_f32(h) for h in vals.split()], np.float32)
        im = np.zeros_like(re)
        codes, scales, _, _ = phasequant_on_gpu(dev(re), dev(im), re.size, 1, want_resid=False)
        torch().cuda.synchronize()
        got = host(scales).view(np.uint32)
        assert got[0] == hex_to_f32(want.strip()).view(np.uint32), line
        assert got[1] == 0


@pytest.mark.parametrize("seed", range(4))
def test_phasequant_wide_dynamic_range(seed):
    """Magnitudes spread over the whole fp32 range in one tensor."""
    g = synth.rng(500 + seed)
    k = 20000
    e = g.integers(-149, 120, size=k).astype(np.float64)
    re = ((g.random(k) + 0.5) * np.exp2(e) * np.where(g.random(k) < 0.5, -1, 1)).astype(np.float32)
    e2 = g.integers(-149, 120, size=k).astype(np.float64)
    im = ((g.random(k) + 0.5) * np.exp2(e2) * np.where(g.random(k) < 0.5, -1, 1)).astype(np.float32)
    _check_pq(re, im, 2)
