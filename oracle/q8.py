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
