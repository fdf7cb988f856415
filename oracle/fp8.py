"""OCP FP8 E4M3FN decoding for the fp8 attention variant.

TEST INFRASTRUCTURE. The decoder is a 256-entry table built from the format
definition (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; there are no infinities and only S.1111.111 is NaN, so
the largest finite magnitude is 1.75 * 2^8 = 448.

The oracle of the fp8 path runs the fp64 attention definition on the decoded
values times their per-(sequence, head) fp32 scale.
"""
from __future__ import annotations

import math

import numpy as np

_BIAS = 7


def decode_code(code: int) -> float:
    """Value of one E4M3FN byte, from the field definition."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - _BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - _BIAS)


E4M3_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes (any shape) -> fp64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes: np.ndarray, scales: np.ndarray, seq_len) -> np.ndarray:
    """Packed [N, H, D] uint8 codes and [nseq, H] fp32 scales -> fp64 [N, H, D].

    Every token of sequence s and head h is multiplied by scales[s, h] in fp64.
    """
    vals = decode(codes)
    out = np.empty_like(vals)
    a = 0
    for s, L in enumerate(seq_len):
        out[a:a + L] = vals[a:a + L] * np.asarray(scales[s], dtype=np.float64)[None, :, None]
        a += L
    return out
