"""Seeded synthetic inputs for the W4A16 matmul.

This module only draws random numbers. It holds none of the method's
arithmetic (no packing, no dequantisation, no products), so that both the
oracle-side tests and the GPU path can take their inputs from it without
sharing any computation.

Recipe (the same for every shape):

* ``numpy.random.default_rng(seed)`` (PCG64), draws taken in this order:
  activations, then weight words, then scales.
* Activations ``A``: ``standard_normal`` in float32, rounded to float16
  (round-to-nearest-even), shape ``[M][K]`` row-major.
* Weight words ``Bq``: uniform ``uint32`` words, shape ``[K/8][N]``.  A word
  holds eight 4-bit codes along K, so uniform words are exactly eight
  independent codes uniform on 0..15.
* Scales ``S``: ``uniform(0.005, 0.02)`` in float64, rounded to float16,
  shape ``[K/group][N]`` row-major.
* Bias (fused output stage only, its own generator): ``standard_normal``
  float32 scaled by ``bias_std``, rounded to float16, shape ``[N]``.
* Zero-point and BF16 formats (``make_inputs_awq``): the same draws in the
  same order, then zero points ``integers(0, 16)`` as uint8
  ``[K/group][N]``.  For BF16 the float32 draws are cut to their upper 16
  bits (truncation, not rounding: a choice of the generator, so that no
  rounding rule is shared with the code under test); values are carried as
  uint16 bit patterns.

* 2:4 masks (``make_mask24``, its own generator): uint8 ``[K/4][N]``.  By
  default each byte is one of the six patterns with exactly two of bits
  0..3 set, uniformly (the pruning the sparse format stores); with
  ``exact=False`` any byte 0..255 (groups with fewer or more set bits, and
  set bits above bit 3).

The value distributions are the ones the workload description gives: a
Gaussian activation, uniform codes, and small positive scales, one per group
of 128 (or one per column when the group is the whole of K).
"""

from __future__ import annotations

import numpy as np

SCALE_LO = 0.005
SCALE_HI = 0.02


def make_inputs(M: int, K: int, N: int, group: int = 128, seed: int = 0):
    """Return ``(A, Bq, S)`` as numpy arrays (float16, uint32, float16)."""
    if K % 8 or group <= 0 or K % group:
        raise ValueError(f"bad shape K={K} group={group}")
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    Bq = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    S = rng.uniform(SCALE_LO, SCALE_HI, size=(K // group, N)).astype(np.float16)
    return A, Bq, S


def make_activations(M: int, K: int, seed: int = 0):
    """Activations alone, ``standard_normal`` float32 rounded to float16."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def make_words(K: int, N: int, seed: int = 0):
    """Uniform ``uint32`` weight words alone, shape ``[K/8][N]``."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)


def make_bias(N: int, seed: int = 0, bias_std: float = 2.0):
    """Per-column bias, ``bias_std * standard_normal`` rounded to float16.

    The default spread is of the order of the products' own (a sum of K
    terms of unit-variance activations and weights of magnitude ~0.05), so
    the activation sees both signs."""
    rng = np.random.default_rng(seed)
    return (bias_std * rng.standard_normal(N, dtype=np.float32)).astype(np.float16)


def make_inputs_awq(M: int, K: int, N: int, group: int = 128, seed: int = 0,
                    bf16: bool = False):
    """Return ``(A, Bq, S, Z)``: as ``make_inputs`` plus uint8 zero points
    ``Z[K/group][N]`` uniform on 0..15.  With ``bf16`` A and S are BF16 bit
    patterns (uint16): the float32 draws with their low 16 bits dropped."""
    if K % 8 or group <= 0 or K % group:
        raise ValueError(f"bad shape K={K} group={group}")
    rng = np.random.default_rng(seed)
    A32 = rng.standard_normal((M, K), dtype=np.float32)
    Bq = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    S64 = rng.uniform(SCALE_LO, SCALE_HI, size=(K // group, N))
    Z = rng.integers(0, 16, size=(K // group, N), dtype=np.uint8)
    if bf16:
        A = (A32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        S = (S64.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    else:
        A = A32.astype(np.float16)
        S = S64.astype(np.float16)
    return A, Bq, S, Z


# The six 4-bit patterns with exactly two bits set, in increasing order.
TWO_OF_FOUR = np.array([0b0011, 0b0101, 0b0110, 0b1001, 0b1010, 0b1100], dtype=np.uint8)


def make_mask24(K: int, N: int, seed: int = 0, exact: bool = True):
    """A 2:4 mask ``uint8[K/4][N]``: uniform over the six two-of-four
    patterns, or (``exact=False``) uniform bytes."""
    if K % 4:
        raise ValueError(f"bad shape K={K}")
    rng = np.random.default_rng(seed)
    if exact:
        return TWO_OF_FOUR[rng.integers(0, 6, size=(K // 4, N), dtype=np.uint8)]
    return rng.integers(0, 256, size=(K // 4, N), dtype=np.uint8)
