"""One fused weight-gradient + optimizer step of a linear layer (oracle).

FORGE explainer, §2 Method, "core mechanism": per weight tile, (1) accumulate
dY/X partial products in FP32 registers, (2) apply the optimizer to the
completed tile, (3) discard the gradient tile, (4) write back only the updated
weight tile and the (optionally quantised) moment tiles. §2 "Precision and
fidelity": for element-wise separable optimizers the tiled update equals a full
gradient step up to the summation order over tokens. The oracle therefore
computes the plain definition: the whole float64 gradient, then the textbook
element-wise update, then the storage formats:

* float32 states and float32 weights: round to nearest float32;
* bfloat16 weights: x32 = round-to-nearest float32 of the float64 result, then
  stochastic rounding with the counter-based r16 (see `rounding`), or
  round-to-nearest-even bfloat16 when stochastic rounding is off;
* INT8 states (linear codes, or the dynamic 8-bit code): dequantise the stored
  codes, update in float64, quantise the new moments (see `q8`). The weight
  update uses the unquantised new moments.
* bfloat16 states: widen the stored values, update in float64, then round like a
  bfloat16 weight (nearest float32, then stochastic rounding with the moment's own
  random stream, or nearest-even when stochastic rounding is off). The weight
  update uses the unrounded new moments.

Row-sampled mode computes the same thing for a subset of output rows only; the
update is element-wise and INT8 blocks never cross rows, so it is the same
oracle on fewer elements.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import fp8, gemm, optim, q8, rounding


def _widen(a: np.ndarray, io: str) -> np.ndarray:
    if io == "bf16":
        return rounding.bf16_to_f64(a)
    if io == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(io)


def _rne_bf16_from_f32(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bits (NaN kept quiet)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x32)
    out = np.where(nan, ((u >> np.uint64(16)) & np.uint64(0x8000)) | np.uint64(0x7FC0), out)
    return out.astype(np.uint16)


def load_state(slot: str, arr: Optional[np.ndarray], scale: Optional[np.ndarray], state: str):
    """Stored moment -> float64 values."""
    if arr is None:
        return None
    if state == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if state == "q8":
        return q8.dequant_signed(arr, scale) if slot == "m" else q8.dequant_sqrt_unsigned(arr, scale)
    if state == "bf16":
        return rounding.bf16_to_f64(arr)
    if state == "q8dyn":
        return q8.dequant_dyn_signed(arr, scale) if slot == "m" else q8.dequant_dyn_unsigned(arr, scale)
    raise ValueError(state)


def store_state(slot: str, val: Optional[np.ndarray], state: str, *, seed: int = 0, t: int = 1,
                idx: Optional[np.ndarray] = None, sr: bool = True):
    """float64 moment -> (stored array, scale or None). bfloat16 states need the
    element indices `idx`, the seed and step for their random stream."""
    if val is None:
        return None, None
    if state == "f32":
        return rounding.rne_f32(val), None
    if state == "bf16":
        x32 = rounding.rne_f32(val)
        if not sr:
            return _rne_bf16_from_f32(x32), None
        stream = rounding.STREAM_M if slot == "m" else rounding.STREAM_V
        return rounding.sr_bf16(x32, rounding.rand16(seed, t, idx, stream)), None
    if state == "q8dyn":
        return q8.quant_dyn_signed(val) if slot == "m" else q8.quant_dyn_unsigned(val)
    if state != "q8":
        raise ValueError(state)
    if slot == "m":
        return q8.quant_signed(val)
    return q8.quant_sqrt_unsigned(val)


def wgrad_step(opt: str, X: np.ndarray, dY: np.ndarray, W: np.ndarray,
               m: Optional[np.ndarray], v: Optional[np.ndarray], hp: Dict[str, float], t: int,
               seed: int, *, io: str = "bf16", state: str = "f32", sr: bool = True,
               rows: Optional[np.ndarray] = None,
               m_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
               g: Optional[np.ndarray] = None, x_fmt: Optional[str] = None, dy_fmt: Optional[str] = None,
               x_scale: float = 1.0, dy_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """One step. With `rows`, W/m/v/scales hold only those output rows.

    X [T, in], dY [T, out] and W are bf16 bit patterns (uint16) when io == "bf16",
    float32 arrays when io == "f32". With x_fmt / dy_fmt ("e4m3" or "e5m2") X / dY
    are uint8 OCP FP8 codes of value code * x_scale / dy_scale (W stays in `io`).
    A precomputed float64 gradient `g` for the selected rows may be passed to avoid
    recomputing it.
    Returns W (stored format), m, v (stored format), m_scale, v_scale, and the
    float64 intermediates g, theta, m64, v64, x32 for tolerance checks.
    """
    n_out = dY.shape[1]
    n_in = X.shape[1]
    rows = np.arange(n_out) if rows is None else np.asarray(rows)
    if g is None:
        Xw = fp8.dequant(X, x_fmt, x_scale) if x_fmt else _widen(X, io)
        dYw = fp8.dequant(dY, dy_fmt, dy_scale) if dy_fmt else _widen(dY, io)
        g = gemm.wgrad_rows(Xw, dYw, rows)
    theta0 = _widen(W, io)
    slots = optim.SLOTS[opt]
    m64 = load_state("m", m, m_scale, state) if "m" in slots else None
    v64 = load_state("v", v, v_scale, state) if "v" in slots else None
    theta, m64n, v64n = optim.update(opt, theta0, g, m64, v64, hp, t)
    idx = rounding.element_index(rows, n_in)
    m_out, ms = store_state("m", m64n, state, seed=seed, t=t, idx=idx, sr=sr)
    v_out, vs = store_state("v", v64n, state, seed=seed, t=t, idx=idx, sr=sr)
    x32 = rounding.rne_f32(theta)
    if io == "f32":
        w_out = x32
    elif sr:
        r16 = rounding.rand16(seed, t, idx)
        w_out = rounding.sr_bf16(x32, r16)
    else:
        w_out = _rne_bf16_from_f32(x32)
    return dict(W=w_out, m=m_out, v=v_out, m_scale=ms, v_scale=vs,
                g=g, theta=theta, m64=m64n, v64=v64n, x32=x32)
