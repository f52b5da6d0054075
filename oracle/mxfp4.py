"""MXFP4 decoding: E2M1 element codes and E8M0 block scales, in float64.

Page: antirez `ds4.c`, `dsv4_e2m1fn_value_cpu` lists the eight E2M1
magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, selected by the low three code bits;
`dsv4_fp4_act_quantize_row_inplace_cpu` groups elements in blocks of 32 that
share one power-of-two scale (2 raised to an integer). Page: goosedump
`gpt_oss.rs`, `validate_tensors`, stores gate/up/down expert weights as
`Mxfp4` tensors.

Readings where the pages are silent (the pages print no MXFP4 byte layout):
- code bit 3 is the sign (the OCP E2M1 layout: s e1 e0 m); code 8 is -0.0;
- a scale byte b means 2^(b - 127); b = 255 is NaN (OCP E8M0);
- codes are packed two per byte, element 2i in the low nibble of byte i.
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    """Closed form of one E2M1 code: sign s, exponent e (2 bits), mantissa m.

    e == 0 is the subnormal 0.5*m; otherwise 2^(e-1) * (1 + m/2).
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else math.ldexp(1.0 + 0.5 * m, e - 1)
    return -mag if s else mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(b: int) -> float:
    """E8M0 block scale: an unbiased power of two, 2^(b-127); 255 is NaN."""
    if b == 255:
        return math.nan
    return math.ldexp(1.0, int(b) - 127)


E8M0 = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2i is the low nibble of byte i."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantise an MXFP4 matrix: w[r, j] = E2M1[code[r, j]] * E8M0[scale[r, j // 32]].

    packed [rows, K/2] uint8, scales [rows, K/32] uint8 -> float64 [rows, K].
    Every value is exactly representable in float32 for scale bytes 1..254
    (the product is E2M1 times a power of two), so `.astype(np.float32)` of
    the result is the bit-exact fp32 weight.
    """
    codes = unpack_codes(packed)
    rows, K = codes.shape[-2], codes.shape[-1]
    if scales.shape[-1] * 32 != K:
        raise ValueError("scale plane does not match K/32")
    vals = E2M1[codes]
    sc = E8M0[np.asarray(scales, dtype=np.uint8)]
    return (vals.reshape(vals.shape[:-1] + (K // 32, 32)) * sc[..., None]).reshape(vals.shape)
