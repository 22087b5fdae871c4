"""Helpers for GPU-vs-oracle parity checks (tolerances written out here).

Tolerances (float point; integer/bit results are exact unless stated):
  * fp32 moments: |gpu - ref| <= 1e-4 * max(|ref|, 0.1 * rms(ref))  (relative 1e-4 with a floor,
    because where dW ~ 0 FP32 accumulation error makes a pure relative bound meaningless).
  * fp32 weights: |gpu - ref| <= 1e-3 * lr per step.
  * bf16 weights with stochastic rounding: bit-exact, except at most 0.01% of elements. Each
    differing element must be explained: its GPU bits must be what the oracle's own step gives
    (same r16) for some gradient within the FP32 summation-error bound of that element,
    |dg| <= T * 2^-24 * sum_t |dY[t,o] X[t,i]| (the pages: the only deviation of the fused step
    is the summation order over tokens), widened by one bfloat16 step for the rounding
    boundary. Where g ~ 0 an adaptive update (m / sqrt(v)) is ill-conditioned and this allows
    more than one step; everywhere else it reduces to "one step at a rounding boundary".
  * INT8 codes: within one quantisation step; scales as fp32 moments.
  * dgrad bf16 output: within one bfloat16 ulp of the float64 value, the ulp taken at
    max(|ref|, 0.01 * rms(ref)).
  * fp32 GEMM outputs (fp32 dgrad, the baseline's stored dW): the a-priori bound of
    floating-point summation in any order, |gpu - ref| <= K * 2^-24 * sum_k |a_k b_k|
    per element (K = length of the contraction).
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


def summation_bound_ok(gpu: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, K: int):
    """(n_bad, worst ratio) for |gpu - ref| <= K * 2^-24 * abs_sum elementwise."""
    bound = K * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64)
    err = np.abs(np.asarray(gpu, dtype=np.float64) - ref)
    return int(np.count_nonzero(err > bound)), float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


def codes_ok(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu.astype(np.int32) - ref.astype(np.int32))
    return int(np.count_nonzero(d > 1)), int(np.count_nonzero(d)), int(d.max()) if d.size else 0


def bf16_step_explained(W_gpu_bits, ref, opt, X, dY, W_b, m_b, v_b, hp, t, seed, io, state, sel,
                        ms_b=None, vs_b=None, frac=1e-4, n_samples=17):
    """(ok, n_diff, n_unexplained, detail) for the bf16 weight check described above."""
    from oracle import step as ostep
    from synth import f32_from_bf16_bits as widen
    d = np.abs(_ordered(W_gpu_bits) - _ordered(ref["W"]))
    bad = np.argwhere(d > 0)
    n = len(bad)
    allowed = max(1, int(np.floor(frac * d.size)))
    Xw = widen(X).astype(np.float64) if io == "bf16" else np.asarray(X, np.float64)
    dYw = widen(dY).astype(np.float64) if io == "bf16" else np.asarray(dY, np.float64)
    T = Xw.shape[0]
    unexplained, detail = 0, []
    for r, i in bad[:200]:
        o = int(sel[r])
        delta = T * 2.0 ** -24 * float(np.sum(np.abs(dYw[:, o] * Xw[:, i])))
        g0 = ref["g"][r].copy()
        cands = []
        for s in np.linspace(-1.0, 1.0, n_samples):
            g = g0.copy()
            g[i] = g0[i] + s * delta
            out = ostep.wgrad_step(opt, X, dY, W_b[r:r + 1],
                                   None if m_b is None else m_b[r:r + 1], None if v_b is None else v_b[r:r + 1],
                                   hp, t, seed, io=io, state=state, rows=np.array([o]),
                                   m_scale=None if ms_b is None else ms_b[r:r + 1],
                                   v_scale=None if vs_b is None else vs_b[r:r + 1], g=g[None, :])
            cands.append(int(_ordered(out["W"][0, i:i + 1])[0]))
        lo, hi = min(cands) - 1, max(cands) + 1
        got = int(_ordered(W_gpu_bits[r, i:i + 1])[0])
        ok_el = lo <= got <= hi
        unexplained += 0 if ok_el else 1
        detail.append((o, int(i), got - int(_ordered(ref["W"][r, i:i + 1])[0]), lo, hi, got, float(g0[i]), delta))
    if n > 200:
        unexplained += n - 200  # only the first 200 are examined; the rest count as unexplained
    return (n <= allowed and unexplained == 0), n, unexplained, detail[:5]


def snapshot(tensors, sel):
    """Host copies of the selected rows of (W, m, v, m_scale, v_scale) (None stays None)."""
    out, idx = [], None
    for t in tensors:
        if t is None:
            out.append(None)
            continue
        if idx is None or idx.device != t.device:
            idx = torch.as_tensor(np.asarray(sel), dtype=torch.long, device=t.device)
        out.append(host(t.index_select(0, idx)))
    return out


def verify_step(opt, X, dY, before, after, hp, t, seed, io, state, sr, sel, g=None):
    """Teacher-forced check of one fused step on the rows `sel` (raises AssertionError).

    before/after: host rows of (W, m, v, m_scale, v_scale) around the GPU step.
    """
    from oracle import step as ostep
    W_b, m_b, v_b, ms_b, vs_b = before
    W_a, m_a, v_a, ms_a, vs_a = after
    ref = ostep.wgrad_step(opt, X, dY, W_b, m_b, v_b, hp, t, seed, io=io, state=state, sr=sr, rows=sel,
                           m_scale=ms_b, v_scale=vs_b, g=g)
    if io == "bf16":
        ok, n, unexplained, detail = bf16_step_explained(W_a, ref, opt, X, dY, W_b, m_b, v_b, hp, t, seed, io,
                                                         state, sel, ms_b, vs_b)
        assert ok, (f"step {t}: {n} of {W_a.size} bf16 weights differ, {unexplained} not explained by a "
                    f"rounding boundary or the FP32 summation bound: {detail}")
    else:
        err = float(np.max(np.abs(W_a.astype(np.float64) - ref["theta"]))) if W_a.size else 0.0
        assert err <= 1e-3 * hp["lr"], f"step {t}: fp32 W error {err}"
    for slot, got, gs in (("m", m_a, ms_a), ("v", v_a, vs_a)):
        if got is None:
            continue
        if state == "f32":
            bad, worst = state_ok(got, ref[slot])
            assert bad == 0, f"step {t}: {slot}: {bad} elements out of tolerance (worst {worst:.3g}x)"
        else:
            big, nd, mx = codes_ok(got, ref[slot])
            assert big == 0, f"step {t}: {slot} codes: {big} off by more than one step"
            bad, worst = state_ok(gs, ref[slot + "_scale"])
            assert bad == 0, f"step {t}: {slot} scales: {bad} out of tolerance (worst {worst:.3g}x)"
    return ref
