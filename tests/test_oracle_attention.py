"""Pins of the oracle's complex attention [iFairy press article §三; Fairy2i
article §2.2; iFairy talk §2.1.4]: the score is the real part of the
Hermitian inner product, equal to the real dot product of the concatenated
real and imaginary parts; the softmax weights average the values' real and
imaginary parts separately."""
import numpy as np
import pytest

import oracle


def rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


def qkv(h, sq, sk, d, seed):
    return [rand(s, seed + i) for i, s in enumerate([(h, sq, d)] * 2 + [(h, sk, d)] * 4)]


def test_score_is_real_dot_product_of_concatenation():
    qr, qi, kr, ki, _, _ = qkv(3, 7, 11, 16, 1)
    s = oracle.cattn_scores(qr, qi, kr, ki, 0.25)
    q2 = np.concatenate([qr, qi], axis=-1).astype(np.float64)
    k2 = np.concatenate([kr, ki], axis=-1).astype(np.float64)
    want = 0.25 * (q2 @ k2.transpose(0, 2, 1))
    assert np.allclose(s, want, rtol=1e-13, atol=1e-13)


def test_score_of_self_is_squared_norm():
    qr, qi, _, _, _, _ = qkv(2, 5, 5, 8, 2)
    s = oracle.cattn_scores(qr, qi, qr, qi, 1.0)
    diag = np.einsum("hii->hi", s)
    want = (qr.astype(np.float64) ** 2 + qi.astype(np.float64) ** 2).sum(-1)
    assert np.allclose(diag, want, rtol=1e-13)


def test_score_symmetric_in_query_and_key():
    """Re(q . conj(k)) = Re(k . conj(q))."""
    qr, qi, kr, ki, _, _ = qkv(1, 6, 6, 12, 3)
    a = oracle.cattn_scores(qr, qi, kr, ki, 1.0)
    b = oracle.cattn_scores(kr, ki, qr, qi, 1.0)
    assert np.allclose(a, b.transpose(0, 2, 1), rtol=1e-13)


def numpy_attention(qr, qi, kr, ki, vr, vi, scale, causal):
    q2 = np.concatenate([qr, qi], axis=-1).astype(np.float64)
    k2 = np.concatenate([kr, ki], axis=-1).astype(np.float64)
    s = scale * (q2 @ k2.transpose(0, 2, 1))
    sq, sk = s.shape[1], s.shape[2]
    if causal:
        mask = np.arange(sk)[None, :] > np.arange(sq)[:, None] + (sk - sq)
        s = np.where(mask[None], -np.inf, s)
    w = np.exp(s - s.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    return w @ vr.astype(np.float64), w @ vi.astype(np.float64)


@pytest.mark.parametrize("h,sq,sk,d,causal", [(2, 5, 9, 8, False), (3, 16, 16, 32, True), (1, 4, 10, 6, True)])
def test_attention_matches_numpy_softmax(h, sq, sk, d, causal):
    qr, qi, kr, ki, vr, vi = qkv(h, sq, sk, d, 10 + sq)
    o_re, o_im = oracle.cattention(qr, qi, kr, ki, vr, vi, 0.3, causal)
    w_re, w_im = numpy_attention(qr, qi, kr, ki, vr, vi, 0.3, causal)
    assert np.allclose(o_re, w_re, rtol=1e-12, atol=1e-12)
    assert np.allclose(o_im, w_im, rtol=1e-12, atol=1e-12)


def test_single_key_returns_its_value():
    qr, qi, kr, ki, vr, vi = qkv(2, 3, 1, 8, 20)
    o_re, o_im = oracle.cattention(qr, qi, kr, ki, vr, vi, 1.0)
    assert np.array_equal(o_re, np.broadcast_to(vr.astype(np.float64), o_re.shape))
    assert np.array_equal(o_im, np.broadcast_to(vi.astype(np.float64), o_im.shape))


def test_zero_query_averages_values():
    _, _, kr, ki, vr, vi = qkv(1, 2, 9, 4, 30)
    z = np.zeros((1, 2, 4), np.float32)
    o_re, o_im = oracle.cattention(z, z, kr, ki, vr, vi, 1.0)
    assert np.allclose(o_re, np.broadcast_to(vr.mean(1, dtype=np.float64)[:, None], o_re.shape), rtol=1e-14)
    assert np.allclose(o_im, np.broadcast_to(vi.mean(1, dtype=np.float64)[:, None], o_im.shape), rtol=1e-14)


def test_causal_rows():
    """Square causal attention: query 0 sees key 0 only; the last query sees all."""
    qr, qi, kr, ki, vr, vi = qkv(1, 6, 6, 4, 40)
    o_re, o_im = oracle.cattention(qr, qi, kr, ki, vr, vi, 0.5, causal=True)
    assert np.array_equal(o_re[0, 0], vr[0, 0].astype(np.float64))
    assert np.array_equal(o_im[0, 0], vi[0, 0].astype(np.float64))
    f_re, f_im = oracle.cattention(qr, qi, kr, ki, vr, vi, 0.5, causal=False)
    assert np.allclose(o_re[0, -1], f_re[0, -1], rtol=1e-14) and np.allclose(o_im[0, -1], f_im[0, -1], rtol=1e-14)
    # with more keys than queries the diagonal shifts by sk - sq
    s = oracle.cattn_scores(qr[:, :2], qi[:, :2], kr, ki, 1.0, causal=True)
    assert np.isinf(s[0, 0, 5]) and np.isfinite(s[0, 0, 4]) and np.isfinite(s[0, 1, 5])


def test_key_permutation_invariance():
    qr, qi, kr, ki, vr, vi = qkv(2, 4, 13, 8, 50)
    perm = np.random.default_rng(5).permutation(13)
    a = oracle.cattention(qr, qi, kr, ki, vr, vi, 0.7)
    b = oracle.cattention(qr, qi, kr[:, perm], ki[:, perm], vr[:, perm], vi[:, perm], 0.7)
    assert np.allclose(a[0], b[0], rtol=1e-13) and np.allclose(a[1], b[1], rtol=1e-13)


def test_sharp_softmax_selects_best_key():
    """A very large scale turns the weights one-hot on the highest score."""
    qr, qi, kr, ki, vr, vi = qkv(1, 3, 7, 4, 60)
    s = oracle.cattn_scores(qr, qi, kr, ki, 1.0)
    o_re, o_im = oracle.cattention(qr, qi, kr, ki, vr, vi, 1e4)
    best = s[0].argmax(-1)
    assert np.allclose(o_re[0], vr[0, best], atol=1e-12) and np.allclose(o_im[0], vi[0, best], atol=1e-12)
