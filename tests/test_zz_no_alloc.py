"""The no-allocation unfused baseline against the workspace one, through the C ABI.

forge_linear_wgrad_unfused_noalloc keeps the float32 dW in the library's static per-GPU
scratch instead of a caller-owned workspace; it runs the same kernels with the same
launch configuration as forge_linear_wgrad_unfused, so the two must agree bit for bit
(stricter than the parity bar of the bf16 path). Two calls in a row, the second on a
smaller layer, and a layer too large for the scratch, which is refused before any launch.
"""
import numpy as np
import pytest
import torch

from oracle import optim
from synth import LayerSpec, draw_layer_batch, draw_layer_init
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _gh(hp):
    return dict(hp, nesterov=int(bool(hp["nesterov"])), stochastic_round=1)


def _pair(f, spec, opt, cfg, step, seed):
    X, dY = draw_layer_batch(cfg, 0, step, spec)
    W0 = draw_layer_init(cfg, 0, spec)
    Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
    hp = optim.hyper(opt)
    runs = []
    for noalloc in (False, True):
        W = P.dev_bf16(W0)
        m, v, _, _ = f.new_states(W, opt, "f32")
        # a non-zero starting state, the same for both runs
        if m is not None:
            m.copy_(torch.linspace(-1e-3, 1e-3, m.numel(), device="cuda").view_as(m))
        if v is not None:
            v.copy_(torch.linspace(0, 1e-6, v.numel(), device="cuda").view_as(v))
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        if noalloc:
            f.wgrad_unfused_noalloc(Xd, dYd, W, m, v, opt, _gh(hp), step, seed)
        else:
            f.wgrad_unfused(Xd, dYd, W, m, v, opt, _gh(hp), step, seed)
        torch.cuda.synchronize()
        if noalloc:
            assert torch.cuda.memory_allocated() == base, "the no-allocation call allocated through torch"
        runs.append((P.host(W), None if m is None else P.host(m), None if v is None else P.host(v)))
    return runs


def test_noalloc_equals_workspace_variant_two_calls():
    import optimizer_gemm_amd as f
    for spec, opt, step in ((LayerSpec("a", 1024, 2048, 520), "adamw", 3), (LayerSpec("b", 256, 512, 130), "nadam", 2)):
        print(f"[case] noalloc vs workspace: {spec.out}x{spec.inn} T={spec.T} {opt} step {step}", flush=True)
        (Wa, ma, va), (Wb, mb, vb) = _pair(f, spec, opt, 77, step, 0x5EED_4242)
        np.testing.assert_array_equal(Wb, Wa)
        for x, y in ((mb, ma), (vb, va)):
            if x is not None:
                np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_noalloc_refuses_a_layer_larger_than_its_scratch():
    import optimizer_gemm_amd as f
    spec = LayerSpec("big", 4104, 4096, 16)            # 4104 * 4096 > 2^24
    W = torch.zeros((spec.out, spec.inn), dtype=torch.bfloat16, device="cuda")
    X = torch.zeros((spec.T, spec.inn), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((spec.T, spec.out), dtype=torch.bfloat16, device="cuda")
    m, v, _, _ = f.new_states(W, "adamw", "f32")
    with pytest.raises(f.ForgeError) as e:
        f.wgrad_unfused_noalloc(X, dY, W, m, v, "adamw", None, 1, 1)
    assert e.value.status == -9
