"""Seeded synthetic inputs for the 2-bit complex linear layer.

The only module shared by the HIP path's tests/benchmark and the CPU oracle.
It draws random numbers and rounds activations to their storage type; it
holds none of the method's arithmetic (no conversion, quantisation, packing
or matmul).

Recipe (NumPy PCG64):
  * real Gaussian: ``standard_normal`` in float64, times sigma, cast to fp32;
  * complex tensors draw the real plane first, then the imaginary plane,
    both row-major;
  * bf16 activations: fp32 N(0,1) rounded to bfloat16, nearest-even;
  * int8 activations: ``integers(-127, 128)`` (so -128 never occurs);
  * seeds: the 256x256 single-GEMV case uses seed 0 for its weights; the
    LLaMA-2-7B-shaped cases use seed = 100 * case + tensor index.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def gaussian(shape, sigma: float, seed: int) -> np.ndarray:
    g = rng(seed)
    return (g.standard_normal(size=shape) * float(sigma)).astype(np.float32)


def complex_gaussian(shape, sigma: float, seed: int):
    """(re, im) fp32 planes, each i.i.d. N(0, sigma^2); re drawn first."""
    g = rng(seed)
    re = (g.standard_normal(size=shape) * float(sigma)).astype(np.float32)
    im = (g.standard_normal(size=shape) * float(sigma)).astype(np.float32)
    return re, im


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs are finite N(0,1) draws."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the fp32 values they denote (exact)."""
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_gaussian(shape, seed: int):
    """(re_bits, im_bits) bf16 planes of N(0,1) draws."""
    re, im = complex_gaussian(shape, 1.0, seed)
    return bf16_bits(re), bf16_bits(im)


def int8_uniform(shape, seed: int):
    """(re, im) int8 planes, uniform in [-127, 127]."""
    g = rng(seed)
    re = g.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
    im = g.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
    return re, im


def random_codes(shape, seed: int) -> np.ndarray:
    """Uniform 2-bit codes (for layout and GEMV tests that need no weights)."""
    return rng(seed).integers(0, 4, size=shape, dtype=np.int64).astype(np.uint8)


def random_scales(planes: int, seed: int) -> np.ndarray:
    """Positive per-plane (s_re, s_im) pairs of mixed magnitude."""
    g = rng(seed)
    return (0.01 + g.random((planes, 2))).astype(np.float32)


# ---------------------------------------------------------------------------
# Named workloads (shapes of the LLaMA-2-7B-sized cases)
# ---------------------------------------------------------------------------
LLAMA7B_PROJ = {
    # name: (real rows, real cols) of the original real layer
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}


def real_layer(rows: int, cols: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """Real weight matrix [rows][cols] ~ N(0, sigma^2), fp32."""
    return gaussian((rows, cols), sigma, seed)
