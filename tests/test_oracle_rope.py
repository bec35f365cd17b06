"""Pins of the oracle's complex rotary position encoding [iFairy press
article §三; iFairy talk §2.1.3]: one complex multiplication per output."""
import numpy as np

import oracle


def rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape), g.standard_normal(shape)


def test_position_zero_is_identity():
    yr, yi = rand((3, 64), 1)
    r, i = oracle.rope(yr, yi, [0, 0, 0], 16, 10000.0)
    assert np.array_equal(r, yr) and np.array_equal(i, yi)


def test_norm_preserved():
    yr, yi = rand((4, 96), 2)
    r, i = oracle.rope(yr, yi, [3, 100, 4095, 17], 32, 10000.0)
    assert np.allclose(r ** 2 + i ** 2, yr ** 2 + yi ** 2, rtol=1e-13)


def test_rotations_compose():
    yr, yi = rand((2, 32), 3)
    a = oracle.rope(*oracle.rope(yr, yi, [5, 70], 32, 500.0), [11, 9], 32, 500.0)
    b = oracle.rope(yr, yi, [16, 79], 32, 500.0)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_scores_depend_on_relative_position():
    """Re(sum q_rot conj(k_rot)) over a head is the same for (p1, p2) and
    (p1 + c, p2 + c): the rotary encoding is relative."""
    qr, qi = rand((1, 64), 4)
    kr, ki = rand((1, 64), 5)

    def score(p1, p2):
        a = oracle.rope(qr, qi, [p1], 64, 10000.0)
        b = oracle.rope(kr, ki, [p2], 64, 10000.0)
        return float(((a[0] + 1j * a[1]) * np.conj(b[0] + 1j * b[1])).real.sum())

    for c in (1, 37, 1000):
        assert abs(score(10, 3) - score(10 + c, 3 + c)) < 1e-10


def test_matches_real_rotate_half():
    """The textbook real rotary embedding of a 2D-dimensional head, pairing
    dimensions (j, j + D), rotates by pos * base^(-2j / 2D)."""
    D, base = 16, 10000.0
    g = np.random.default_rng(6)
    x = g.standard_normal((3, 2 * D))
    pos = np.array([0, 7, 1234])
    inv_freq = base ** (-np.arange(0, 2 * D, 2) / (2 * D))
    ang = pos[:, None] * inv_freq[None, :]
    x1, x2 = x[:, :D], x[:, D:]
    want = np.concatenate([x1 * np.cos(ang) - x2 * np.sin(ang), x1 * np.sin(ang) + x2 * np.cos(ang)], axis=1)
    r, i = oracle.rope(x1, x2, pos, D, base)
    assert np.allclose(np.concatenate([r, i], axis=1), want, rtol=1e-12, atol=1e-12)


def test_first_dimension_turns_one_radian_per_position():
    yr = np.ones((1, 8))
    yi = np.zeros((1, 8))
    r, i = oracle.rope(yr, yi, [3], 8, 10000.0)
    assert np.isclose(r[0, 0], np.cos(3.0), rtol=1e-15) and np.isclose(i[0, 0], np.sin(3.0), rtol=1e-15)
    assert np.isclose(r[0, 0] ** 2 + i[0, 0] ** 2, 1.0)
