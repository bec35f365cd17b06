"""GPU parity of the fused complex attention against the fp64 oracle on the
same bf16 inputs: relative L2 error <= 1e-5, the float bound of the layer
itself (fairy.h: exact scores, weights carried as bf16 hi + lo pairs to
~2^-17 relative precision, fp32 accumulation; measured errors 1.3e-6 to
2.3e-6)."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, log, rel_l2, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5


def make(h, sq, sk, d, seed):
    bits, vals = [], []
    for i, (n_) in enumerate([sq, sq, sk, sk, sk, sk]):
        b = synth.bf16_bits(synth.gaussian((h, n_, d), 1.0, seed + i))
        bits.append(b)
        vals.append(synth.bf16_to_f32(b))
    return bits, vals


def run(bits, h, sq, sk, d, scale, causal):
    t = torch()
    o_re = t.empty((h, sq, d), dtype=t.float32, device="cuda")
    o_im = t.empty_like(o_re)
    F.fairy_cattention(*[dev(b) for b in bits], F.FAIRY_BF16, h, sq, sk, d, scale, causal, o_re, o_im)
    t.cuda.synchronize()
    return host(o_re), host(o_im)


CASES = [
    # (heads, sq, sk, d, causal)
    (2, 64, 64, 64, 0),
    (2, 64, 64, 64, 1),
    (3, 50, 77, 32, 0),          # ragged queries and keys
    (1, 37, 100, 128, 1),        # causal with more keys than queries
    (2, 1, 300, 64, 0),          # one query (decode)
    (1, 130, 130, 64, 1),        # three query blocks, three key chunks
    (4, 5, 1, 32, 0),            # a single key: o = v
    (1, 200, 260, 128, 0),
    (2, 257, 1000, 64, 1),       # causal, two query blocks per head, ragged tail chunk
    (1, 129, 640, 32, 0),        # keys a whole number of chunks, ragged queries
    (1, 300, 333, 128, 1),
]


@pytest.mark.parametrize("h,sq,sk,d,causal", CASES)
def test_cattention(h, sq, sk, d, causal):
    log(f"cattention h={h} sq={sq} sk={sk} d={d} causal={causal}")
    bits, v = make(h, sq, sk, d, 100 + sq + sk)
    scale = 1.0 / np.sqrt(2 * d)
    o_re, o_im = run(bits, h, sq, sk, d, scale, causal)
    w_re, w_im = oracle.cattention(*v, scale, bool(causal))
    err = rel_l2(o_re + 1j * o_im, w_re + 1j * w_im)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("scale,causal,sk", [(1.0, 0, 192), (3.0, 1, 700)])
def test_cattention_sharp_scores(scale, causal, sk):
    """Scores spread over tens of units: the running maximum moves by more
    than the lazy threshold mid-sequence, so the output rescaling and the
    exp of large negative arguments are exercised."""
    h, sq, d = 2, 64 if not causal else 300, 64
    log(f"cattention sharp scale={scale} causal={causal} sk={sk}")
    bits, v = make(h, sq, sk, d, 77)
    o_re, o_im = run(bits, h, sq, sk, d, scale, causal)
    w_re, w_im = oracle.cattention(*v, scale, bool(causal))
    err = rel_l2(o_re + 1j * o_im, w_re + 1j * w_im)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("scale,causal", [(-0.3, 0), (-1.0, 1), (0.0, 1)])
def test_cattention_negative_and_zero_scale(scale, causal):
    """A negative scale favours the lowest scores (applied as a positive one
    to the negated queries); a zero scale weights every visible key equally."""
    h, sq, sk, d = 2, 70, 130, 64
    log(f"cattention scale={scale} causal={causal}")
    bits, v = make(h, sq, sk, d, 55)
    o_re, o_im = run(bits, h, sq, sk, d, scale, causal)
    w_re, w_im = oracle.cattention(*v, scale, bool(causal))
    err = rel_l2(o_re + 1j * o_im, w_re + 1j * w_im)
    log(f"  rel_l2={err:.3e}")
    assert err <= TOL


def test_cattention_llama_prefill_sampled_heads():
    """LLaMA-2-7B attention at prefill: 32 heads, 2048 tokens, real head dim
    128 (complex d = 64), causal; the oracle checks heads 0 and 31."""
    h, s, d = 32, 2048, 64
    log("cattention 32 x 2048 x 64 causal")
    bits, v = make(h, s, s, d, 900)
    scale = 1.0 / np.sqrt(2 * d)
    o_re, o_im = run(bits, h, s, s, d, scale, 1)
    for hh in (0, 31):
        w_re, w_im = oracle.cattention(*[x[hh:hh + 1] for x in v], scale, True)
        err = rel_l2(o_re[hh] + 1j * o_im[hh], w_re[0] + 1j * w_im[0])
        log(f"  head {hh} rel_l2={err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_cattention_long_sequence_sampled(d):
    """8192 tokens, causal: the first and last 64 queries against the oracle
    (the first see keys 0..63 only; the last see all keys up to themselves,
    so the oracle on those queries with every key reproduces them)."""
    h, s = 2, 8192
    log(f"cattention long sequence h={h} s={s} d={d}")
    bits, v = make(h, s, s, d, 1000 + d)
    scale = 1.0 / np.sqrt(2 * d)
    o_re, o_im = run(bits, h, s, s, d, scale, 1)
    q_re, q_im, k_re, k_im, v_re, v_im = v
    w_re, w_im = oracle.cattention(q_re[:, :64], q_im[:, :64], k_re[:, :64], k_im[:, :64], v_re[:, :64],
                                   v_im[:, :64], scale, True)
    err = rel_l2(o_re[:, :64] + 1j * o_im[:, :64], w_re + 1j * w_im)
    log(f"  first 64: rel_l2={err:.3e}")
    assert err <= TOL
    w_re, w_im = oracle.cattention(q_re[:, -64:], q_im[:, -64:], k_re, k_im, v_re, v_im, scale, True)
    err = rel_l2(o_re[:, -64:] + 1j * o_im[:, -64:], w_re + 1j * w_im)
    log(f"  last 64: rel_l2={err:.3e}")
    assert err <= TOL


def test_cattention_deterministic():
    h, sq, sk, d = 2, 100, 100, 64
    bits, _ = make(h, sq, sk, d, 5)
    a = run(bits, h, sq, sk, d, 0.1, 1)
    b = run(bits, h, sq, sk, d, 0.1, 1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
