"""INT8 block-64 absmax codec for optimizer moments (oracle).

The pages say the INT8 optimizer states use blocks of 64 elements instead of
the 2048 of standard 8-bit optimizers, to keep quantisation error small (§2
"Precision and fidelity", low-precision fidelity list; one page prints "2024",
read as 2048). They give no codebook. Reading used here: linear absmax codes
on blocks of 64 consecutive elements along a row of the [out, in] state, one
float32 scale per block (scales are [out, in/64]):

* first moment m (signed):  s = max|m| / 127,  q = clamp(rne(m / s), -127, 127)  (int8),
  value q * s.
* second moment v (>= 0), stored through its square root r = sqrt(v):
  s = max r / 255,  q = clamp(rne(r / s), 0, 255)  (uint8),  value (q * s)**2.
  Quantising v itself linearly maps most small v of a block to 0 while m stays
  non-zero, which makes m / (sqrt(v) + eps) explode; the square root keeps the
  dynamic range (a reading, stated as such).
* an all-zero block has s = 0 and q = 0.
The scale is stored as float32; codes are computed from the float32 scale.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

BLOCK = 64


def _blocks(x: np.ndarray, block: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % block:
        raise ValueError("row length must be a multiple of the block size")
    return x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))


def quant_signed(m: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """m -> (int8 codes [.., n], float32 scales [.., n/block])."""
    xb = _blocks(m, block)
    s32 = (np.max(np.abs(xb), axis=-1) / 127.0).astype(np.float32)
    s = s32.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(xb / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(np.shape(m)), s32


def dequant_signed(q: np.ndarray, s32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    qb = _blocks(q.astype(np.float64), block)
    return (qb * s32.astype(np.float64)[..., None]).reshape(q.shape)


def quant_sqrt_unsigned(v: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """v (>= 0) -> (uint8 codes of sqrt(v), float32 scales)."""
    r = np.sqrt(np.maximum(np.asarray(v, dtype=np.float64), 0.0))
    rb = _blocks(r, block)
    s32 = (np.max(rb, axis=-1) / 255.0).astype(np.float32)
    s = s32.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(rb / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, 255).astype(np.uint8)
    return q.reshape(np.shape(v)), s32


def dequant_sqrt_unsigned(q: np.ndarray, s32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    qb = _blocks(q.astype(np.float64), block)
    r = qb * s32.astype(np.float64)[..., None]
    return (r * r).reshape(q.shape)


# ---------------------------------------------------------------------------
# Dynamic (non-linear) 8-bit code on blocks of 64 — the other reading of the
# pages' INT8 states: the "standard 8-bit optimizers" the pages compare against
# store moments in a dynamic-exponent 8-bit code normalised by the block absmax
# (Dettmers et al., "8-bit Optimizers via Block-wise Quantization", dynamic tree
# quantization). That description fixes the layout of a code but not its exact
# values; the construction below is this project's own reading of it:
#
# * a code's magnitude bits hold, from the top, a run of E zeros (the decade),
#   an indicator 1, then F fraction bits f; with n magnitude bits F = n - 1 - E;
# * magnitude = 10^-E * (0.1 + 0.9 (f + 1) / 2^F), i.e. the exact rational
#   (2^F + 9 (f + 1)) / (2^F 10^(E + 1)); the all-zero magnitude is 0.
#   Each decade [10^-(E+1), 10^-E] holds 2^F codes, the largest being 10^-E, so
#   the all-ones code is exactly 1 and the smallest non-zero one 10^-(n-1);
# * signed (m): byte = sign << 7 | k with a 7-bit magnitude index k (0x80 decodes
#   to 0 like 0x00 and is never written); unsigned (v): byte = 8-bit index k;
# * the float32 table value of k is the double quotient N / D rounded to float32;
# * encoding: the block scale is s = max|x| over the float32 moments of the block;
#   y = x / s in float32; the magnitude index is the number of float32 midpoints
#   (v_k + v_k+1) / 2 (rounded to float32) that are <= |y| — the nearest code, ties
#   to the larger; a zero block has s = 0 and codes 0. Decoded value = v_k * s.
# The second moment is coded directly (the dynamic range of the code keeps small v
# of a block non-zero down to 10^-7 of its absmax).
# ---------------------------------------------------------------------------


def dyn_table(n_bits: int) -> np.ndarray:
    """float32 magnitudes of the 2^n_bits magnitude indices, ascending."""
    vals = [0.0]
    for k in range(1, 1 << n_bits):
        F = k.bit_length() - 1          # the indicator bit's position
        E = (n_bits - 1) - F            # zeros above it
        f = k - (1 << F)
        num = (1 << F) + 9 * (f + 1)
        den = (1 << F) * 10 ** (E + 1)
        vals.append(float(np.float32(np.float64(num) / np.float64(den))))
    return np.array(vals, dtype=np.float32)


def dyn_midpoints(table: np.ndarray) -> np.ndarray:
    t = table.astype(np.float64)
    return ((t[:-1] + t[1:]) * 0.5).astype(np.float32)


DYN_SIGNED = dyn_table(7)      # 128 magnitudes for m
DYN_UNSIGNED = dyn_table(8)    # 256 magnitudes for v
_MID_S = dyn_midpoints(DYN_SIGNED)
_MID_U = dyn_midpoints(DYN_UNSIGNED)


def _block_scale32(x32: np.ndarray, block: int) -> np.ndarray:
    xb = x32.reshape(x32.shape[:-1] + (x32.shape[-1] // block, block))
    return np.max(np.abs(xb), axis=-1).astype(np.float32)


def _normalised(x32: np.ndarray, s32: np.ndarray, block: int) -> np.ndarray:
    """float32 x / s per block (0 where s == 0)."""
    xb = x32.reshape(x32.shape[:-1] + (x32.shape[-1] // block, block))
    s = s32[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(s > 0, xb / np.where(s > 0, s, np.float32(1)), np.float32(0)).astype(np.float32)
    return y.reshape(x32.shape)


def quant_dyn_signed(m: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """m -> (uint8 sign-magnitude dynamic codes, float32 block absmax scales)."""
    x32 = np.asarray(m, dtype=np.float64).astype(np.float32)
    _blocks(x32, block)
    s32 = _block_scale32(x32, block)
    y = _normalised(x32, s32, block)
    k = np.searchsorted(_MID_S, np.abs(y), side="right").astype(np.uint8)
    neg = (y < 0) & (k > 0)
    return (k | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8), s32


def dequant_dyn_signed(q: np.ndarray, s32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    qb = np.asarray(q).view(np.uint8) if np.asarray(q).dtype == np.int8 else np.asarray(q, dtype=np.uint8)
    mag = DYN_SIGNED[qb & 0x7F].astype(np.float64)
    val = np.where(qb & 0x80, -mag, mag)
    return (_blocks(val, block) * s32.astype(np.float64)[..., None]).reshape(qb.shape)


def quant_dyn_unsigned(v: np.ndarray, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """v (>= 0) -> (uint8 dynamic codes, float32 block max scales)."""
    x32 = np.maximum(np.asarray(v, dtype=np.float64), 0.0).astype(np.float32)
    _blocks(x32, block)
    s32 = _block_scale32(x32, block)
    y = _normalised(x32, s32, block)
    k = np.searchsorted(_MID_U, y, side="right").astype(np.uint8)
    return k, s32


def dequant_dyn_unsigned(q: np.ndarray, s32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    val = DYN_UNSIGNED[np.asarray(q, dtype=np.uint8)].astype(np.float64)
    return (_blocks(val, block) * s32.astype(np.float64)[..., None]).reshape(np.shape(q))


def dyn_rank(q: np.ndarray, signed: bool) -> np.ndarray:
    """Position of a code in value order (signed: -k for negative codes)."""
    b = np.asarray(q).view(np.uint8).astype(np.int32) if np.asarray(q).dtype == np.int8 \
        else np.asarray(q, dtype=np.uint8).astype(np.int32)
    if not signed:
        return b
    return np.where(b & 0x80, -(b & 0x7F), b & 0x7F)
