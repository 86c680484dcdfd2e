"""Decoding of OCP FP8 E4M3 ("e4m3fn") codes. TEST INFRASTRUCTURE ONLY.

The pages run the model in FP8 on an H100 ([MC-zh] capabilities list); the
format is not named there. The reading taken is the OCP 8-bit floating point
specification's E4M3 encoding (the one gfx950 decodes natively): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2**-6; the all-ones exponent with all-ones mantissa is NaN;
there are no infinities (the largest finite magnitude is 448).
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """The real value of one E4M3 code (0..255), from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """Elementwise decode of a uint8 array of E4M3 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes, scale) -> np.ndarray:
    """codes [..., K] times a per-row scale [...] (float64)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]
