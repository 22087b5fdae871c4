"""Training-step integration: a linear layer whose backward pass performs its own update.

FORGE (explainer pages, §2 Method) folds the optimizer step into the weight-
gradient computation of the backward pass; the input gradient must be read
before the weights change (§5, limitations). ForgeLinear wires that into
PyTorch autograd: forward is Y = X W^T; backward computes dX = dY W with the
library's dgrad kernel on the current (old) W, then enqueues the fused
wgrad + optimizer kernel on the same stream, which updates W and its moments in
place. The weight gradient is never materialised: backward returns None for it,
so `weight.grad` stays None and no optimizer.step() follows.

Each backward call is one optimizer step of that layer (a module used several
times per step, such as a tied embedding, is outside what the method supports).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import forge

_SEED_MIX = 0x9E3779B97F4A7C15


class _ForgeLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, layer: "ForgeLinear") -> torch.Tensor:
        ctx.layer = layer
        ctx.save_for_backward(x)
        # forward product (not part of the fused path): a plain library GEMM
        return torch.matmul(x, weight.t())

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        (x,) = ctx.saved_tensors
        layer: ForgeLinear = ctx.layer
        w = layer.weight
        x2 = x.reshape(-1, w.shape[1])
        dy2 = dy.reshape(-1, w.shape[0])
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        if not dy2.is_contiguous() or dy2.dtype != w.dtype:
            dy2 = dy2.to(w.dtype).contiguous()
        dx = None
        if ctx.needs_input_grad[0]:
            dx = forge.dgrad(dy2, w.detach()).reshape(x.shape)  # old W, before the update below
        layer._step_count += 1
        forge.wgrad_step(x2, dy2, w.detach(), layer.m, layer.v, layer.opt, layer.hyper, layer._step_count,
                         layer.seed, layer.m_scale, layer.v_scale, code=layer.code)
        return dx, None, None


class ForgeLinear(torch.nn.Module):
    """Y = X W^T with the optimizer step fused into the backward pass.

    weight: [out, in] bf16 or float32 parameter (bias-free, as the linear
    layers the pages evaluate). opt / hyper: the optimizer and its
    hyper-parameters (forge_hyper fields). states: "f32", "bf16", "q8" (INT8
    block-64, linear codes) or "q8dyn" (INT8 block-64, dynamic 8-bit code).
    """

    def __init__(self, in_features: int, out_features: int, opt: str = "adamw", hyper: Optional[dict] = None,
                 states: str = "f32", dtype: torch.dtype = torch.bfloat16, device=None, seed: int = 0,
                 weight: Optional[torch.Tensor] = None):
        super().__init__()
        if weight is None:
            weight = torch.empty(out_features, in_features, dtype=dtype, device=device)
            torch.nn.init.normal_(weight, std=0.02)
        self.weight = torch.nn.Parameter(weight, requires_grad=True)
        self.opt = opt
        self.hyper = forge.make_hyper(opt, **(hyper or {}))
        m, v, ms, vs = forge.new_states(self.weight.detach(), opt, states)
        self.code = "dynamic" if states == "q8dyn" else "linear"
        for name, t in (("m", m), ("v", v), ("m_scale", ms), ("v_scale", vs)):
            if t is None:
                setattr(self, name, None)
            else:
                self.register_buffer(name, t)
        self.seed = (int(seed) * _SEED_MIX) & (2 ** 64 - 1)
        self._step_count = 0

    @property
    def step_count(self) -> int:
        return self._step_count

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return _ForgeLinearFn.apply(x, self.weight, self)
