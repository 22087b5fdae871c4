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

For comparison the same module runs the usual two-phase schedule with
fused=False: backward stores the float32 dW (the "gradient floor" every layer
holds until the optimizer runs) and `step_all(model)` then applies the update
with the library's stand-alone optimizer pass. Both schedules use the same
kernels and the same per-element update, so they differ only in when the
gradient exists and where it lives.
"""
from __future__ import annotations

from typing import Optional

import torch
import torch.utils.checkpoint

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
        if not layer.fused:
            # two-phase schedule: the float32 gradient waits for step_all(); a second
            # backward before it adds to it, as the usual gradient accumulation does
            g = forge.wgrad(x2, dy2)
            if layer.grad32 is None:
                layer.grad32 = g
            else:
                layer.grad32.add_(g)
            return dx, None, None
        layer._step_count += 1
        ev = layer.timing
        if ev is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        forge.wgrad_step(x2, dy2, w.detach(), layer.m, layer.v, layer.opt, layer.hyper, layer._step_count,
                         layer.seed, layer.m_scale, layer.v_scale, code=layer.code)
        if ev is not None:
            e1.record()
            ev.append((e0, e1))
        return dx, None, None


class ForgeLinear(torch.nn.Module):
    """Y = X W^T with the optimizer step fused into the backward pass.

    weight: [out, in] bf16 or float32 parameter (bias-free, as the linear
    layers the pages evaluate). opt / hyper: the optimizer and its
    hyper-parameters (forge_hyper fields). states: "f32", "bf16", "q8" (INT8
    block-64, linear codes) or "q8dyn" (INT8 block-64, dynamic 8-bit code).
    fused: True for the fused step in backward; False for the two-phase schedule
    (float32 gradient kept in `grad32`, update applied by `step()`).
    timing: if a list, each fused call appends its (start, end) CUDA events.
    """

    def __init__(self, in_features: int, out_features: int, opt: str = "adamw", hyper: Optional[dict] = None,
                 states: str = "f32", dtype: torch.dtype = torch.bfloat16, device=None, seed: int = 0,
                 weight: Optional[torch.Tensor] = None, fused: bool = True):
        super().__init__()
        self.fused = bool(fused)
        self.grad32: Optional[torch.Tensor] = None
        self.timing: Optional[list] = None
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

    def step(self) -> None:
        """Two-phase schedule: apply the optimizer to the stored gradient and free it
        (nothing to do for a fused layer, whose backward already stepped)."""
        if self.fused or self.grad32 is None:
            return
        self._step_count += 1
        forge.optimizer_step(self.grad32, self.weight.detach(), self.m, self.v, self.opt, self.hyper,
                             self._step_count, self.seed, self.m_scale, self.v_scale, code=self.code)
        self.grad32 = None


class _ForgeGroupFn(torch.autograd.Function):
    """Several ForgeLinear layers applied to the same input: forward Y_l = X W_l^T for each;
    backward dX = sum_l dY_l W_l (each on the old W_l) and then one grouped fused step of
    all the layers (forge_linear_wgrad_step_group), where the layers' tiles share the
    launch."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, layers, *weights: torch.Tensor):
        ctx.layers = layers
        ctx.save_for_backward(x)
        return tuple(torch.matmul(x, w.t()) for w in weights)

    @staticmethod
    def backward(ctx, *dys):
        (x,) = ctx.saved_tensors
        layers = ctx.layers
        ws = [L.weight.detach() for L in layers]
        x2 = x.reshape(-1, ws[0].shape[1])
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        dy2s = []
        for w, dy in zip(ws, dys):
            if dy is None:  # an output that reached no loss: a zero gradient, the layer still steps
                dy2s.append(torch.zeros((x2.shape[0], w.shape[0]), dtype=w.dtype, device=w.device))
                continue
            dy2 = dy.reshape(-1, w.shape[0])
            dy2s.append(dy2 if dy2.is_contiguous() and dy2.dtype == w.dtype else dy2.to(w.dtype).contiguous())
        dx = None
        if ctx.needs_input_grad[0]:
            dx = forge.dgrad(dy2s[0], ws[0])  # old W, before the update below
            for w, dy2 in zip(ws[1:], dy2s[1:]):
                dx.add_(forge.dgrad(dy2, w))
            dx = dx.reshape(x.shape)
        L0 = layers[0]
        if not L0.fused:
            for L, dy2 in zip(layers, dy2s):
                g = forge.wgrad(x2, dy2)
                if L.grad32 is None:
                    L.grad32 = g
                else:
                    L.grad32.add_(g)
            return (dx, None) + (None,) * len(layers)
        for L in layers:
            L._step_count += 1
        ev = L0.timing
        if ev is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        forge.wgrad_step_group(x2, dy2s, ws, [L.m for L in layers], [L.v for L in layers], L0.opt, L0.hyper,
                               L0._step_count, [L.seed for L in layers], [L.m_scale for L in layers],
                               [L.v_scale for L in layers], code=L0.code)
        if ev is not None:
            e1.record()
            ev.append((e0, e1))
        return (dx, None) + (None,) * len(layers)


def grouped_linear(layers, x: torch.Tensor):
    """Y_l = X W_l^T for ForgeLinear layers that read the same input x, as one autograd node
    whose backward steps all of them in one grouped launch (the layers' outputs as a tuple).
    The layers must agree in optimizer, hyper-parameters, moment format, schedule and step
    count; the group's time is recorded on the first layer's `timing` list."""
    layers = list(layers)
    L0 = layers[0]
    if not 1 <= len(layers) <= forge.MAX_GROUP:
        raise ValueError(f"a group holds 1..{forge.MAX_GROUP} layers")
    for L in layers[1:]:
        if (L.opt, L.code, L.fused, L._step_count, L.weight.dtype) != (L0.opt, L0.code, L0.fused, L0._step_count,
                                                                         L0.weight.dtype) or \
                (L.m is None) != (L0.m is None) or (L.v is None) != (L0.v is None) or \
                (L.m is not None and L.m.dtype != L0.m.dtype) or \
                any(getattr(L.hyper, n) != getattr(L0.hyper, n) for n, _ in L0.hyper._fields_):
            raise ValueError("grouped layers must share optimizer, hyper-parameters, states, schedule and step")
    return _ForgeGroupFn.apply(x, layers, *[L.weight for L in layers])


def step_all(model: torch.nn.Module) -> None:
    """The optimizer phase of the two-phase schedule for every ForgeLinear in `model`."""
    for mod in model.modules():
        if isinstance(mod, ForgeLinear):
            mod.step()


def _rms_norm(x: torch.Tensor, eps: float = 1e-5) -> torch.Tensor:
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(x.dtype)


class SwiGLUBlock(torch.nn.Module):
    """Residual SwiGLU MLP block of a Llama-style decoder layer built from ForgeLinear:
    y = x + down(silu(gate(n(x))) * up(n(x))), with n a parameter-free RMS norm.
    gate / up: [hidden, d] weights, down: [d, hidden]. With checkpoint=True the block
    keeps only its input for backward and recomputes the rest (activation
    checkpointing); the recomputation runs before any of the block's layers steps,
    so it sees the same weights as the forward pass. With grouped=True gate and up, which
    read the same n(x), take their fused steps in one grouped launch."""

    def __init__(self, d: int, hidden: int, checkpoint: bool = False, seed: int = 0, grouped: bool = False, **kw):
        super().__init__()
        self.gate = ForgeLinear(d, hidden, seed=3 * seed, **kw)
        self.up = ForgeLinear(d, hidden, seed=3 * seed + 1, **kw)
        self.down = ForgeLinear(hidden, d, seed=3 * seed + 2, **kw)
        self.checkpoint = checkpoint
        self.grouped = grouped

    def _body(self, x: torch.Tensor) -> torch.Tensor:
        h = _rms_norm(x)
        if self.grouped:
            g, u = grouped_linear((self.gate, self.up), h)
        else:
            g, u = self.gate(h), self.up(h)
        return x + self.down(torch.nn.functional.silu(g) * u)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if self.checkpoint and torch.is_grad_enabled():
            return torch.utils.checkpoint.checkpoint(self._body, x, use_reentrant=False)
        return self._body(x)
