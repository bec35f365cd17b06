"""Pins for the oracle's packing (16 two-bit codes per uint32).

The pages fix only the 2-bit code ([Fairy2i article §3.1]; 2 bits per
weight, [iFairy press article §一]); the two word layouts are this library's
own definitions (include/fairy.h).  Pinned against hand-evaluated words and
round trips.
"""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import synth
from tests._golden import rows


def test_golden_words():
    n = 0
    for line in rows("pack_words.txt"):
        head, codes = line.split(";")
        layout, m, word, want = head.split()
        c = np.array([int(t) for t in codes.split()], np.uint8).reshape(1, 1, int(m))
        words = oracle.pack(c, int(layout))
        assert "%08x" % words[int(word)] == want, line
        n += 1
    assert n >= 12


@pytest.mark.parametrize("layout", [oracle.ROW16, oracle.TILED64])
@pytest.mark.parametrize("planes,rows_,m", [(1, 3, 16), (4, 5, 80), (2, 7, 256), (6, 2, 5504)])
def test_round_trip(layout, planes, rows_, m):
    c = synth.random_codes((planes, rows_, m), 17)
    w = oracle.pack(c, layout)
    assert w.size == oracle.packed_words(rows_, m, planes, layout)
    assert np.array_equal(oracle.unpack(w, planes, rows_, m, layout), c)
    # density: exactly 2 bits per code (plus zero padding to 64 columns in TILED64)
    ones = sum(bin(int(x)).count("1") for x in w)
    assert ones == int(sum(bin(int(x)).count("1") for x in c.ravel()))


def test_tiled_padding_is_code0():
    c = np.full((1, 1, 16), 3, np.uint8)
    w = oracle.pack(c, oracle.TILED64)
    assert w.size == 4 and w[0] == 0xFFFFFFFF and not w[1:].any()


def test_tiled_plane_interleave():
    """Word ((r*G + g)*P + p)*4 + u holds plane p's columns 64g+16u..+15."""
    P, R, m = 3, 2, 128
    c = np.zeros((P, R, m), np.uint8)
    c[2, 1, 64 + 16 * 3 + 1] = 1          # plane 2, row 1, group 1, word 3, t = 1
    w = oracle.pack(c, oracle.TILED64)
    idx = ((1 * 2 + 1) * P + 2) * 4 + 3
    assert w[idx] == 1 << 30 and np.count_nonzero(w) == 1
