"""Helpers for GPU-vs-oracle parity checks (tolerances written out here).

Tolerances (float point; integer/bit results are exact unless stated):
  * fp32 moments: |gpu - ref| <= 1e-4 * max(|ref|, 0.1 * rms(ref))  (relative 1e-4 with a floor,
    because where dW ~ 0 FP32 accumulation error makes a pure relative bound meaningless).
  * fp32 weights: |gpu - ref| <= 1e-3 * lr per step.
  * bf16 weights with stochastic rounding: bit-exact, except at most 0.01% of elements that
    may sit one bfloat16 step away (their float32 value lies within the GPU/oracle arithmetic
    difference of a rounding boundary).
  * INT8 codes: within one quantisation step; scales as fp32 moments.
  * dgrad bf16 output: within one bfloat16 ulp of the float64 value, the ulp taken at
    max(|ref|, 0.01 * rms(ref)); fp32 output: 1e-5 relative with the same kind of floor.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import f32_from_bf16_bits


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev(arr: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return host_bits(t)
    return t.detach().cpu().numpy()


def state_ok(gpu: np.ndarray, ref: np.ndarray, rel: float = 1e-4, floor: float = 0.1):
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * np.maximum(np.abs(ref), floor * rms)
    err = np.abs(gpu - ref)
    bad = err > bound
    return int(bad.sum()), float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_sr_ok(gpu_bits: np.ndarray, ref_bits: np.ndarray, frac: float = 1e-4):
    """(ok, n_diff, max_step_distance)."""
    d = np.abs(_ordered(gpu_bits) - _ordered(ref_bits))
    n = int(np.count_nonzero(d))
    mx = int(d.max()) if d.size else 0
    allowed = max(1, int(np.floor(frac * d.size)))
    return (mx <= 1 and n <= allowed), n, mx


def dgrad_bf16_ok(gpu_bits: np.ndarray, ref64: np.ndarray):
    g = f32_from_bf16_bits(gpu_bits).astype(np.float64)
    rms = float(np.sqrt(np.mean(ref64 * ref64))) if ref64.size else 0.0
    mag = np.maximum(np.abs(ref64), 0.01 * rms)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 7)
    err = np.abs(g - ref64)
    return int(np.count_nonzero(err > ulp)), float(np.max(err / ulp)) if err.size else 0.0


def codes_ok(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu.astype(np.int32) - ref.astype(np.int32))
    return int(np.count_nonzero(d > 1)), int(np.count_nonzero(d)), int(d.max()) if d.size else 0
