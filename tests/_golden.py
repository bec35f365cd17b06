"""Readers for the hand-worked fixtures under tests/golden/ and exact
rational helpers used by the oracle pins."""
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield line


def hex_to_f32(h: str) -> np.float32:
    return np.frombuffer(struct.pack("<I", int(h, 16)), np.float32)[0]


def f32_to_hex(x) -> str:
    return "%08x" % struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def exact_f32_round(q: Fraction) -> np.float32:
    """Nearest fp32 to the non-negative rational q, ties to even significand,
    decided by exact rational distances (independent of the oracle's C code)."""
    assert q >= 0
    f0 = np.float32(float(q))
    cands = {f0, np.nextafter(f0, np.float32(0)), np.nextafter(f0, np.float32(np.inf))}
    best = None
    for c in sorted(cands):
        if c < 0 or not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])
