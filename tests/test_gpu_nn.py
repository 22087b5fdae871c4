"""GPU tests of the training-step integration (ForgeLinear).

The backward pass of a two-layer MLP built from ForgeLinear must (1) leave no
weight gradient behind, (2) compute each input gradient from the old weights,
and (3) update every weight exactly as a direct call of the fused step with
that layer's (X, dY) would; the last layer's update is also checked against
the oracle.
"""
import numpy as np
import pytest
import torch

from oracle import optim
from tests import _parity as P

pytestmark = pytest.mark.gpu


def test_forge_linear_mlp_step_matches_direct_calls():
    import optimizer_gemm_amd as forge
    from optimizer_gemm_amd.nn import ForgeLinear

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    T, d_in, d_hid, d_out = 200, 256, 512, 128
    l1 = ForgeLinear(d_in, d_hid, device=dev, seed=1)
    l2 = ForgeLinear(d_hid, d_out, device=dev, seed=2)
    W1_0, W2_0 = l1.weight.detach().clone(), l2.weight.detach().clone()
    x = torch.randn(T, d_in, device=dev, generator=g).to(torch.bfloat16).requires_grad_(True)
    G = (torch.randn(T, d_out, device=dev, generator=g) * 1e-3).to(torch.bfloat16)

    h = l1(x)
    a = torch.nn.functional.gelu(h)
    y = l2(a)
    y.backward(G)
    torch.cuda.synchronize()
    assert l1.weight.grad is None and l2.weight.grad is None
    assert l1.step_count == 1 and l2.step_count == 1

    # reference: the same kernels called directly, in the order the method requires
    W2 = W2_0.clone()
    m2, v2, _, _ = forge.new_states(W2, "adamw")
    dA = forge.dgrad(G, W2_0)                       # input gradient from the old W2
    forge.wgrad_step(a.detach(), G, W2, m2, v2, "adamw", None, 1, l2.seed)
    h_ref = h.detach().requires_grad_(True)
    (dH,) = torch.autograd.grad(torch.nn.functional.gelu(h_ref), h_ref, dA)
    W1 = W1_0.clone()
    m1, v1, _, _ = forge.new_states(W1, "adamw")
    dX = forge.dgrad(dH.contiguous(), W1_0)
    forge.wgrad_step(x.detach(), dH.contiguous(), W1, m1, v1, "adamw", None, 1, l1.seed)
    torch.cuda.synchronize()
    assert torch.equal(l2.weight.detach().view(torch.int16), W2.view(torch.int16))
    assert torch.equal(l2.m, m2) and torch.equal(l2.v, v2)
    assert torch.equal(l1.weight.detach().view(torch.int16), W1.view(torch.int16))
    assert torch.equal(x.grad.view(torch.int16), dX.view(torch.int16))

    # and the last layer's step against the oracle
    hp = optim.hyper("adamw")
    sel = np.arange(d_out)
    before = [P.host_bits(W2_0), np.zeros((d_out, d_hid), np.float32), np.zeros((d_out, d_hid), np.float32),
              None, None]
    after = [P.host_bits(l2.weight.detach()), P.host(l2.m), P.host(l2.v), None, None]
    P.verify_step("adamw", P.host_bits(a.detach()), P.host_bits(G), before, after, hp, 1, l2.seed, "bf16", "f32",
                  True, sel)


def test_forge_linear_no_gradient_memory():
    # the backward pass allocates dX but never a weight-sized gradient
    from optimizer_gemm_amd.nn import ForgeLinear

    dev = torch.device("cuda:0")
    layer = ForgeLinear(2048, 2048, device=dev, seed=3)
    x = torch.randn(64, 2048, device=dev).to(torch.bfloat16)
    y = layer(x)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    y.backward(torch.ones_like(y) * 1e-3)
    torch.cuda.synchronize()
    grown = torch.cuda.max_memory_allocated() - base
    assert layer.weight.grad is None
    assert grown < 2048 * 2048 * 2  # well below one bf16 weight gradient


@pytest.mark.parametrize("states", ["q8", "q8dyn", "bf16"])
def test_forge_linear_low_precision_states_match_direct_calls(states):
    # a ForgeLinear with INT8 (linear or dynamic codes) or bf16 moments updates W and its
    # moments exactly as the direct call with the same state format does
    import optimizer_gemm_amd as forge
    from optimizer_gemm_amd.nn import ForgeLinear

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(6)
    T, d_in, d_out = 160, 256, 192
    print(f"[case] ForgeLinear states={states}", flush=True)
    layer = ForgeLinear(d_in, d_out, device=dev, seed=4, states=states)
    W0 = layer.weight.detach().clone()
    x = torch.randn(T, d_in, device=dev, generator=g).to(torch.bfloat16)
    G = (torch.randn(T, d_out, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    layer(x).backward(G)
    W = W0.clone()
    m, v, ms, vs = forge.new_states(W, "adamw", states)
    forge.wgrad_step(x, G, W, m, v, "adamw", None, 1, layer.seed, ms, vs, code=P.state_code(states))
    torch.cuda.synchronize()
    assert torch.equal(layer.weight.detach().view(torch.int16), W.view(torch.int16))
    for a, b in ((layer.m, m), (layer.v, v), (layer.m_scale, ms), (layer.v_scale, vs)):
        assert (a is None and b is None) or torch.equal(a, b)


def _mlp_model(fused, ckpt, d, hidden, blocks, dev):
    from optimizer_gemm_amd.nn import SwiGLUBlock
    torch.manual_seed(21)
    return torch.nn.Sequential(*[SwiGLUBlock(d, hidden, checkpoint=ckpt, seed=b, fused=fused, device=dev)
                                 for b in range(blocks)])


def _train(model, x, G, steps, fused):
    from optimizer_gemm_amd.nn import step_all
    grads = []
    for _ in range(steps):
        xin = x.clone().requires_grad_(True)
        model(xin).backward(G)
        if not fused:
            step_all(model)
        grads.append(xin.grad)
    torch.cuda.synchronize()
    return grads


def _lin_state(model):
    from optimizer_gemm_amd.nn import ForgeLinear
    return [(m.weight.detach().clone(), m.m.clone(), m.v.clone()) for m in model.modules()
            if isinstance(m, ForgeLinear)]


def test_checkpointed_block_equals_plain_block():
    # activation checkpointing recomputes each block's forward before any of its layers
    # steps, so weights, moments and the input gradient are bit-identical to the run
    # that keeps its activations
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(8)
    T, d, hidden = 192, 256, 640
    print("[case] SwiGLU blocks, checkpoint on/off", flush=True)
    x = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
    G = (torch.randn(T, d, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    runs = []
    for ckpt in (False, True):
        model = _mlp_model(True, ckpt, d, hidden, 2, dev)
        grads = _train(model, x, G, 3, True)
        runs.append((_lin_state(model), grads))
    (s0, g0), (s1, g1) = runs
    for (w0, m0, v0), (w1, m1, v1) in zip(s0, s1):
        assert torch.equal(w0.view(torch.int16), w1.view(torch.int16))
        assert torch.equal(m0, m1) and torch.equal(v0, v1)
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("ckpt", [False, True])
def test_grouped_gate_up_equals_separate_layers(ckpt):
    # gate and up (same input) as one grouped launch: dX is the sum of the two dgrads on
    # the old weights, as autograd sums the separate layers' contributions, and on these
    # shapes the grouped and the single-layer launchers pick the same 64x128 tiles, so
    # weights, moments and input gradients equal the ungrouped block's bit for bit
    from optimizer_gemm_amd.nn import SwiGLUBlock
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(9)
    T, d, hidden = 256, 256, 512
    print(f"[case] SwiGLU blocks, gate/up grouped vs separate, checkpoint={ckpt}", flush=True)
    x = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
    G = (torch.randn(T, d, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    runs = []
    for grouped in (False, True):
        torch.manual_seed(21)
        model = torch.nn.Sequential(*[SwiGLUBlock(d, hidden, checkpoint=ckpt, seed=b, grouped=grouped, device=dev)
                                      for b in range(2)])
        grads = _train(model, x, G, 3, True)
        runs.append((_lin_state(model), grads, [m.step_count for m in model.modules() if hasattr(m, "step_count")]))
    (s0, g0, c0), (s1, g1, c1) = runs
    assert c0 == c1 == [3] * len(c0)
    for (w0, m0, v0), (w1, m1, v1) in zip(s0, s1):
        assert torch.equal(w0.view(torch.int16), w1.view(torch.int16))
        assert torch.equal(m0, m1) and torch.equal(v0, v1)
    for a, b in zip(g0, g1):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_two_phase_schedule_matches_fused():
    # the two-phase schedule (float32 dW stored in backward, optimizer pass afterwards)
    # and the fused one apply the same update: at step 1 bit for bit up to the SR flips the
    # tolerance of the unfused comparison allows, and the step-1 input gradients are equal
    from optimizer_gemm_amd.nn import ForgeLinear
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(9)
    T, d, hidden = 160, 256, 512
    print("[case] SwiGLU block, fused vs two-phase", flush=True)
    x = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
    G = (torch.randn(T, d, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    res = []
    for fused in (True, False):
        model = _mlp_model(fused, False, d, hidden, 1, dev)
        grads = _train(model, x, G, 1, fused)
        lins = [m for m in model.modules() if isinstance(m, ForgeLinear)]
        assert all(m.weight.grad is None and m.grad32 is None and m.step_count == 1 for m in lins)
        res.append((_lin_state(model), grads))
    (sf, gf), (st, gt) = res
    assert torch.equal(gf[0].view(torch.int16), gt[0].view(torch.int16))
    for (wf, mf, vf), (wt, mt, vt) in zip(sf, st):
        ok, n, mx = P.bf16_sr_ok(P.host_bits(wf), P.host_bits(wt))
        assert ok, (n, mx)
        assert P.state_ok(P.host(mf), P.host(mt), rel=1e-6)[0] == 0
        assert P.state_ok(P.host(vf), P.host(vt), rel=1e-6)[0] == 0


def test_two_phase_peak_memory_holds_the_gradient_floor():
    # the two-phase step holds the float32 gradients of every layer (4 bytes per weight) at
    # once at the end of backward, when the activations are already freed; the fused
    # schedule never allocates them, so its peak is the activations and input gradients
    from optimizer_gemm_amd.nn import step_all
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(10)
    T, d, hidden, blocks = 256, 1024, 2816, 2
    print("[case] SwiGLU blocks, peak memory fused vs two-phase", flush=True)
    x = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
    G = (torch.randn(T, d, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
    peaks = {}
    for fused in (True, False):
        model = _mlp_model(fused, False, d, hidden, blocks, dev)
        xin = x.clone().requires_grad_(True)
        # one step first: the first GEMMs of a process allocate library workspaces
        model(xin).backward(G)
        if not fused:
            step_all(model)
        xin.grad = None
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        model(xin).backward(G)
        if not fused:
            step_all(model)
        torch.cuda.synchronize()
        peaks[fused] = torch.cuda.max_memory_allocated() - base
        del model, xin
        torch.cuda.empty_cache()
    floor = blocks * 3 * 4 * d * hidden
    assert peaks[False] >= floor, (peaks, floor)
    assert peaks[True] < 0.5 * floor, (peaks, floor)
