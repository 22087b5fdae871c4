"""Counter-based random numbers and stochastic rounding to bfloat16 (oracle).

The pages say only that the bfloat16 weight write-back uses stochastic rounding
so that sub-ULP updates accumulate without bias and the bfloat16 "dead zone" is
avoided (§2 "Precision and fidelity", low-precision fidelity list). They give no
generator and no rounding rule. Reading used here (fully specified so both sides
can reproduce it bit for bit):

* Counter  c = (t << 32) | idx, t the 1-based step, idx = o*in + i the row-major
  index of the weight element (independent of any tiling).
* Random 64-bit word: the (c+1)-th output of SplitMix64 started from state
  `seed` (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): z = seed + (c+1)*0x9E3779B97F4A7C15 (mod 2**64), then the
  SplitMix64 finaliser. r16 = z >> 48.
* bfloat16 moment states are rounded the same way with other 16-bit fields of
  the same 64-bit word: bits 32..47 for m, bits 16..31 for v (the weight takes
  bits 48..63), so one SplitMix64 evaluation serves all three roundings of an
  element.
* Stochastic rounding of a float32 x: bf16 bits = (bits(x) + r16) >> 16 on the
  unsigned 32-bit pattern, which rounds the magnitude away from zero with
  probability low16(bits(x)) / 65536. NaN becomes the quiet NaN 0x7FC0 with the
  sign kept; +-Inf and -0 are preserved by the formula itself.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1


def splitmix64_py(seed: int, n: int):
    """First n SplitMix64 outputs from state `seed`, with Python integers (mod 2**64)."""
    s = seed & _M64
    out = []
    for _ in range(n):
        s = (s + GOLDEN_GAMMA) & _M64
        z = s
        z = ((z ^ (z >> 30)) * MIX1) & _M64
        z = ((z ^ (z >> 27)) * MIX2) & _M64
        out.append(z ^ (z >> 31))
    return out


def splitmix64_at(seed: int, counter: np.ndarray) -> np.ndarray:
    """The (counter+1)-th SplitMix64 output from state `seed`, vectorised (uint64)."""
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _M64) + (c + np.uint64(1)) * np.uint64(GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        z = z ^ (z >> np.uint64(31))
    return z


def counters(step: int, idx: np.ndarray) -> np.ndarray:
    """c = (step << 32) | idx; idx must be < 2**32."""
    idx = np.asarray(idx, dtype=np.uint64)
    if idx.size and int(idx.max()) >= (1 << 32):
        raise ValueError("element index must fit in 32 bits")
    return (np.uint64(step) << np.uint64(32)) | idx


STREAM_W, STREAM_M, STREAM_V = 0, 1, 2


def rand16(seed: int, step: int, idx: np.ndarray, stream: int = STREAM_W) -> np.ndarray:
    """16 random bits per element (uint32 array): bits 48..63 of the SplitMix64 word
    for the weight (stream 0), bits 32..47 for m (1), bits 16..31 for v (2)."""
    if stream not in (STREAM_W, STREAM_M, STREAM_V):
        raise ValueError(stream)
    z = splitmix64_at(seed, counters(step, idx))
    return ((z >> np.uint64(48 - 16 * stream)) & np.uint64(0xFFFF)).astype(np.uint32)


def element_index(rows: np.ndarray, n_in: int) -> np.ndarray:
    """Row-major idx = o*in + i for the given output rows and all in columns."""
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    cols = np.arange(n_in, dtype=np.uint64).reshape(1, -1)
    return rows * np.uint64(n_in) + cols


def rne_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def sr_bf16(x32: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Stochastic rounding of float32 values to bfloat16 bits (uint16) with given r16."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = np.asarray(r16, dtype=np.uint64)
    out = ((u + r) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x32)
    if np.any(nan):
        sign = (u >> np.uint64(16)) & np.uint64(0x8000)
        out = np.where(nan, sign | np.uint64(0x7FC0), out)
    return out.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
