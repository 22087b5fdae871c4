"""Weight gradient and input gradient of a linear layer, in float64.

FORGE explainer, §2 Method, "core mechanism": for a weight tile the kernel
accumulates partial products of the upstream gradient dY and the input
activation X over the tokens. The plain definition of that sum for a layer
Y = X W^T (W is [out, in], X is [T, in], dY is [T, out]) is
    dW[o, i] = sum_t dY[t, o] * X[t, i]        (summed over tokens, not averaged)
and the input gradient (limitations paragraph: it is read before the weight
update, i.e. uses the old W) is
    dX[t, i] = sum_o dY[t, o] * W[o, i].
bfloat16 and float32 inputs widen exactly to float64, so with float64
accumulation the products are exact and only the summation rounds.
"""
from __future__ import annotations

import numpy as np


def wgrad(X: np.ndarray, dY: np.ndarray) -> np.ndarray:
    """dW = dY^T X in float64; X [T, in], dY [T, out] -> [out, in]."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    if X.ndim != 2 or dY.ndim != 2 or X.shape[0] != dY.shape[0]:
        raise ValueError("X [T,in] and dY [T,out] must share T")
    return dY.T @ X


def wgrad_rows(X: np.ndarray, dY: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Rows `rows` of dW only: dY[:, rows]^T X. Same definition on a subset."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    return dY[:, rows].T @ X


def wgrad_tiled(X: np.ndarray, dY: np.ndarray, tile_o: int = 128, tile_i: int = 128,
                chunk_t: int = 64) -> np.ndarray:
    """dW assembled tile by tile, each tile accumulated over token chunks.

    This is the schedule the pages describe (one weight tile at a time, partial
    products summed into the tile's accumulator); it must agree with `wgrad`
    up to summation order (§2 "Precision and fidelity", exactness paragraph).
    """
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    T, n_in = X.shape
    n_out = dY.shape[1]
    out = np.empty((n_out, n_in), dtype=np.float64)
    for o0 in range(0, n_out, tile_o):
        for i0 in range(0, n_in, tile_i):
            acc = np.zeros((min(tile_o, n_out - o0), min(tile_i, n_in - i0)))
            for t0 in range(0, T, chunk_t):
                acc += dY[t0:t0 + chunk_t, o0:o0 + tile_o].T @ X[t0:t0 + chunk_t, i0:i0 + tile_i]
            out[o0:o0 + tile_o, i0:i0 + tile_i] = acc
    return out


def dgrad(dY: np.ndarray, W: np.ndarray) -> np.ndarray:
    """dX = dY W in float64; dY [T, out], W [out, in] -> [T, in]."""
    dY = np.asarray(dY, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if dY.shape[1] != W.shape[0]:
        raise ValueError("dY [T,out] and W [out,in] must share out")
    return dY @ W
