"""Decoding of OCP 8-bit floating point inputs (oracle).

FORGE's pages name FP8 inputs as compatible with the fused step (§5, outlook) and
give no format; the reading here is the two OCP 8-bit formats ("OCP 8-bit Floating
Point Specification (OFP8)", Open Compute Project, 2023) that gfx950's matrix cores
take, each tensor carrying one float32 dequantisation scale:

* E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
  subnormal (mantissa * 2^-9); no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.
* E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent 0 is
  subnormal (mantissa * 2^-16); exponent 31 holds +-infinity (mantissa 0) and NaN.

value(code, scale) = decode(code) * scale, in float64.
"""
from __future__ import annotations

import numpy as np

FORMATS = ("e4m3", "e5m2")
_BITS = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}  # exponent bits, mantissa bits, bias


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """float64 values of uint8 codes in the given OCP format."""
    if fmt not in _BITS:
        raise ValueError(fmt)
    eb, mb, bias = _BITS[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    mant = c & ((1 << mb) - 1)
    frac = mant / float(1 << mb)
    val = np.where(e == 0, frac * 2.0 ** (1 - bias), (1.0 + frac) * np.exp2(e - bias))
    if fmt == "e4m3":
        val = np.where((e == 15) & (mant == 7), np.nan, val)
    else:
        val = np.where(e == 31, np.where(mant == 0, np.inf, np.nan), val)
    return sign * val


def dequant(codes: np.ndarray, fmt: str, scale: float) -> np.ndarray:
    """decode(codes) * scale with the tensor's float32 scale, in float64."""
    return decode(codes, fmt) * float(np.float32(scale))
