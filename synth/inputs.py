"""Seeded synthetic workloads for the fused weight-gradient + optimizer step.

The pages evaluate on Llama-3.1-8B and Qwen3 layers (FORGE explainer, section 4
"Experimental results"); no dataset or trained weight is used here. Every tensor
is drawn from numpy's PCG64 generator seeded by
``SeedSequence([0xF06E, config, layer, step, tensor_id])`` with
tensor_id 0 = W init, 1 = X, 2 = dY, 3 = X outlier rows, 4 = dY outlier rows.
Dense tensors are drawn in chunks of whole rows (about 4M values each); chunk k
uses the same seed sequence extended by k, so the values do not depend on the
number of threads that fill them. "N(0, s)" means standard deviation s.
bfloat16 tensors are the round-to-nearest-even bfloat16 of the float32 sample,
done on the bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_TAG = 0xF06E
TID_W, TID_X, TID_DY, TID_X_OUT, TID_DY_OUT = 0, 1, 2, 3, 4


_THREADS = max(1, min(16, os.cpu_count() or 1))
_CHUNK = 1 << 22


def layer_seed(config: int, layer: int, step: int, tensor_id: int) -> np.random.Generator:
    """PCG64 generator for one tensor of one layer at one step."""
    ss = np.random.SeedSequence([ROOT_TAG, int(config), int(layer), int(step), int(tensor_id)])
    return np.random.Generator(np.random.PCG64(ss))


def _row_chunks(rows: int, cols: int):
    step = max(1, _CHUNK // max(cols, 1))
    return [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]


def _parallel(fn, n):
    if n <= 1:
        for k in range(n):
            fn(k)
        return
    with ThreadPoolExecutor(max_workers=min(_THREADS, n)) as ex:
        list(ex.map(fn, range(n)))


def _bf16_rne_inplace(x: np.ndarray, out: np.ndarray) -> None:
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # < 2**32 for every finite float32
    r >>= np.uint32(16)
    out[...] = r


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bfloat16 (nearest, ties to even); returns uint16 bits.

    Only finite samples occur in these workloads; NaN or Inf inputs are rejected.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.ndim < 2:
        flat_x, flat_o = x.reshape(1, -1), out.reshape(1, -1)
    else:
        flat_x, flat_o = x.reshape(-1, x.shape[-1]), out.reshape(-1, x.shape[-1])
    chunks = _row_chunks(flat_x.shape[0], flat_x.shape[1])
    bad = [False] * len(chunks)

    def work(k):
        r0, r1 = chunks[k]
        if not np.all(np.isfinite(flat_x[r0:r1])):
            bad[k] = True
            return
        _bf16_rne_inplace(flat_x[r0:r1], flat_o[r0:r1])

    _parallel(work, len(chunks))
    if any(bad):
        raise ValueError("synthetic inputs must be finite")
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_normal(key: Tuple[int, ...], shape: Tuple[int, int], std: float) -> np.ndarray:
    """float32 N(0, std) samples of a 2-D tensor; `key` = (config, layer, step, tensor_id)."""
    rows, cols = shape
    x = np.empty((rows, cols), dtype=np.float32)
    chunks = _row_chunks(rows, cols)

    def work(k):
        r0, r1 = chunks[k]
        ss = np.random.SeedSequence([ROOT_TAG] + [int(v) for v in key] + [k])
        np.random.Generator(np.random.PCG64(ss)).standard_normal(out=x[r0:r1], dtype=np.float32)
        if std != 1.0:
            x[r0:r1] *= np.float32(std)

    _parallel(work, len(chunks))
    return x


def outlier_rows(config: int, layer: int, step: int, tensor_id: int, T: int, frac: float) -> np.ndarray:
    """Sorted, distinct token rows chosen as outliers: round(frac * T) of them."""
    n = int(round(frac * T))
    gen = layer_seed(config, layer, step, tensor_id)
    return np.sort(gen.choice(T, size=n, replace=False))


def sample_rows(config: int, layer: int, out: int, n: int) -> np.ndarray:
    """Seeded subset of output rows for row-sampled parity checks (sorted, distinct)."""
    n = min(n, out)
    gen = layer_seed(config, layer, 0, 99)
    return np.sort(gen.choice(out, size=n, replace=False))


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer: W is [out, in]; X is [T, in]; dY is [T, out]."""
    name: str
    out: int
    inn: int
    T: int
    io: str = "bf16"              # "bf16" or "f32" for X, dY and W
    w_std: float = 0.02
    x_std: float = 1.0
    dy_std: float = 1e-3
    outlier_frac: float = 0.0     # fraction of token rows scaled by outlier_scale
    outlier_scale: float = 100.0

    @property
    def P(self) -> int:
        return self.out * self.inn


def _to_io(x32: np.ndarray, io: str) -> np.ndarray:
    return bf16_bits_from_f32(x32) if io == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def draw_layer_init(config: int, layer: int, spec: LayerSpec) -> np.ndarray:
    """Initial W (uint16 bf16 bits or float32)."""
    w = draw_normal((config, layer, 0, TID_W), (spec.out, spec.inn), spec.w_std)
    return _to_io(w, spec.io)


def draw_layer_batch(config: int, layer: int, step: int, spec: LayerSpec) -> Tuple[np.ndarray, np.ndarray]:
    """Fresh (X, dY) for one step (step is 1-based); bf16 bits or float32."""
    x = draw_normal((config, layer, step, TID_X), (spec.T, spec.inn), spec.x_std)
    dy = draw_normal((config, layer, step, TID_DY), (spec.T, spec.out), spec.dy_std)
    if spec.outlier_frac > 0.0:
        rx = outlier_rows(config, layer, step, TID_X_OUT, spec.T, spec.outlier_frac)
        rd = outlier_rows(config, layer, step, TID_DY_OUT, spec.T, spec.outlier_frac)
        x[rx, :] *= np.float32(spec.outlier_scale)
        dy[rd, :] *= np.float32(spec.outlier_scale)
    return _to_io(x, spec.io), _to_io(dy, spec.io)


FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def fp8_codes(x: np.ndarray, fmt: str) -> Tuple[np.ndarray, float]:
    """Per-tensor scaled OCP FP8 codes of float32 data: scale = absmax / largest finite
    value of the format (1 for an all-zero tensor), codes = round-to-nearest-even of
    x / scale (PyTorch's conversion). Returns (uint8 codes, float32 scale)."""
    import torch
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(amax / FP8_MAX[fmt]) if amax > 0 else np.float32(1.0)
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    q = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / scale).to(dt)
    return q.view(torch.uint8).numpy().copy(), float(scale)


def draw_layer_batch_fp8(config: int, layer: int, step: int, spec: LayerSpec, x_fmt: str = "e4m3",
                         dy_fmt: str = "e5m2") -> Tuple[np.ndarray, np.ndarray, float, float]:
    """The same (X, dY) draw as draw_layer_batch, as FP8 codes with per-tensor scales:
    (X codes, dY codes, x scale, dY scale)."""
    x = draw_normal((config, layer, step, TID_X), (spec.T, spec.inn), spec.x_std)
    dy = draw_normal((config, layer, step, TID_DY), (spec.T, spec.out), spec.dy_std)
    if spec.outlier_frac > 0.0:
        rx = outlier_rows(config, layer, step, TID_X_OUT, spec.T, spec.outlier_frac)
        rd = outlier_rows(config, layer, step, TID_DY_OUT, spec.T, spec.outlier_frac)
        x[rx, :] *= np.float32(spec.outlier_scale)
        dy[rd, :] *= np.float32(spec.outlier_scale)
    xq, sx = fp8_codes(x, x_fmt)
    dq, sd = fp8_codes(dy, dy_fmt)
    return xq, dq, sx, sd


def _llama8b_layers(T: int) -> List[LayerSpec]:
    h, kv, ff = 4096, 1024, 14336
    return [
        LayerSpec("q_proj", h, h, T), LayerSpec("k_proj", kv, h, T), LayerSpec("v_proj", kv, h, T),
        LayerSpec("o_proj", h, h, T), LayerSpec("gate_proj", ff, h, T), LayerSpec("up_proj", ff, h, T),
        LayerSpec("down_proj", h, ff, T),
    ]


def _llama8b_tp8_layers(T: int) -> List[LayerSpec]:
    """One GPU's shards of the seven linears under 8-way tensor parallelism: the
    column-parallel ones (q, k, v, gate, up) split `out`, the row-parallel ones (o,
    down) split `in`; every GPU sees all T tokens."""
    h, kv, ff, tp = 4096, 1024, 14336, 8
    return [
        LayerSpec("q_proj", h // tp, h, T), LayerSpec("k_proj", kv // tp, h, T), LayerSpec("v_proj", kv // tp, h, T),
        LayerSpec("o_proj", h, h // tp, T), LayerSpec("gate_proj", ff // tp, h, T), LayerSpec("up_proj", ff // tp, h, T),
        LayerSpec("down_proj", h, ff // tp, T),
    ]


@dataclass
class Workload:
    """A named workload: its layers, optimizer(s), step count and state format."""
    config: int
    name: str
    layers: List[LayerSpec]
    steps: int
    optimizers: Tuple[str, ...] = ("adamw",)
    state: str = "f32"                 # "f32" or "q8" (int8 m, uint8 sqrt-v, block 64)
    stochastic_round: bool = True
    extra: Dict[str, object] = field(default_factory=dict)


WORKLOADS: Dict[str, Workload] = {
    # fp32 everything, 256x256, 512 tokens, AdamW, 3 steps, no stochastic rounding
    "fp32_256": Workload(0, "fp32_256", [LayerSpec("linear", 256, 256, 512, io="f32", dy_std=1e-2)],
                         steps=3, stochastic_round=False),
    # q_proj-shaped: 4096x4096 bf16, 8192 tokens, AdamW + SR, 10 steps
    "q_proj_8192": Workload(1, "q_proj_8192", [LayerSpec("q_proj", 4096, 4096, 8192)], steps=10),
    # the seven linears of a Llama-3.1-8B-shaped decoder layer, 8192 tokens
    "llama8b_layer_8192": Workload(2, "llama8b_layer_8192", _llama8b_layers(8192), steps=1),
    # INT8 block-64 states on down_proj, 16384 tokens, 1% outlier rows x100, 20 steps
    "down_q8_16384": Workload(3, "down_q8_16384",
                              [LayerSpec("down_proj", 4096, 14336, 16384, outlier_frac=0.01)],
                              steps=20, state="q8"),
    # eight optimizers on a Qwen3-14B-shaped MLP weight 17408x5120, 4096 tokens, 10 steps
    "qwen14b_mlp_4096": Workload(4, "qwen14b_mlp_4096", [LayerSpec("mlp_up", 17408, 5120, 4096)], steps=10,
                                 optimizers=("adamw", "nadam", "radam", "lion", "rmsprop", "adagrad",
                                             "sgd", "sgd_momentum")),
    # one GPU's 8-way tensor-parallel shards of the Llama-3.1-8B-shaped layer, 8192 tokens
    "llama8b_tp8_8192": Workload(6, "llama8b_tp8_8192", _llama8b_tp8_layers(8192), steps=1),
}


def llama8b_stack(T: int = 8192, n_layers: int = 32) -> List[LayerSpec]:
    """All 7*n_layers linear layers of an n_layers-deep Llama-8B-shaped stack."""
    out: List[LayerSpec] = []
    for _ in range(n_layers):
        out.extend(_llama8b_layers(T))
    return out
