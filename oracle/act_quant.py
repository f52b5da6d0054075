"""MX-FP4 round trip of activations (blocks of 32 values sharing one
power-of-two scale, E2M1 elements), as the quantised expert-input mode uses it.

Page: antirez `ds4.c`, `dsv4_fp4_act_quantize_row_inplace_cpu` and
`dsv4_e2m1fn_dequant_cpu`. Per block of 32 consecutive values the page
  1. takes the largest magnitude amax, held at no less than 6 * 2^-126;
  2. takes the scale 2^ceil(log2(amax / 6)), so amax / scale <= 6;
  3. divides each value by the scale and clamps it to [-6, 6];
  4. replaces its magnitude by the nearest E2M1 magnitude
     {0, 0.5, 1, 1.5, 2, 3, 4, 6}; at an equal distance the even code index
     wins (the index with a zero mantissa bit);
  5. keeps the sign of the value (a value that is not below zero, -0.0
     included, is positive) and multiplies back by the scale.

Reading where the page leaves a step open: step 2 is taken exactly, as the
smallest integer e with amax <= 6 * 2^e (from amax's own exponent and
mantissa bits). The page evaluates it with float32 log2f and ceilf, which
agree with this except where log2f rounds a quotient just above a power of
two down onto it; there the page would use half this scale and clamp the
block maximum to 6.

Element codes follow the weights' E2M1 layout (bit 3 the sign, bits 0-2 the
magnitude index); the scale is the E8M0 byte e + 127.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .mxfp4 import E2M1

MAGS = E2M1[:8].copy()            # 0, 0.5, 1, 1.5, 2, 3, 4, 6
AMAX_FLOOR = 6.0 * 2.0 ** -126    # the page's lower bound on a block's amax


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 6 * 2^e, for float32 amax >= 6 * 2^-126.

    amax = m * 2^E with m in [1, 2): 6 * 2^(E-2) = 1.5 * 2^E >= amax exactly
    when m <= 1.5, else e = E - 1 (6 * 2^(E-1) = 3 * 2^E > amax)."""
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    E = ((bits >> 23) & 0xFF) - 127
    mant = bits & 0x7FFFFF
    return np.where(mant <= 0x400000, E - 2, E - 1)


def nearest_index(v: np.ndarray) -> np.ndarray:
    """Index (0..7) of the E2M1 magnitude nearest to |v| (|v| <= 6), ties to
    the even index: candidates are taken in index order, and a later one
    replaces the current choice when strictly nearer, or equally near with an
    even index against an odd current one."""
    av = np.abs(np.asarray(v, dtype=np.float64))
    best = np.zeros(av.shape, dtype=np.int64)
    best_d = np.abs(av - MAGS[0])
    for i in range(1, 8):
        d = np.abs(av - MAGS[i])
        take = (d < best_d) | ((d == best_d) & (i % 2 == 0) & (best % 2 == 1))
        best = np.where(take, i, best)
        best_d = np.where(take, d, best_d)
    return best


def quantize_rows(x: np.ndarray):
    """Round trip of float32 rows [..., K] (K a multiple of 32).

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32], values
    float64 [..., K] = sign * E2M1 magnitude * 2^e, each exact in float32)."""
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    if K % 32:
        raise ValueError("rows must hold whole 32-value blocks")
    blk = x.reshape(x.shape[:-1] + (K // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)                             # step 1
    amax = np.maximum(amax, np.float32(AMAX_FLOOR))
    e = block_exponent(amax)                                         # step 2
    scale = np.ldexp(1.0, e)[..., None]
    v = np.clip(blk.astype(np.float64) / scale, -6.0, 6.0)           # step 3
    idx = nearest_index(v)                                           # step 4
    neg = blk < 0                                                    # step 5
    codes = (idx | np.where(neg, 8, 0)).astype(np.uint8)
    vals = np.where(neg, -MAGS[idx], MAGS[idx]) * scale
    return (codes.reshape(x.shape), (e + 127).astype(np.uint8), vals.reshape(x.shape))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes -> [..., K/2] bytes, element 2i in the low nibble of byte i
    (the weights' packing)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
