"""The layer step captured in a HIP graph and replayed, against the same calls made eagerly.

A training loop that launches the same layers every step can capture dgrad and the fused
step once and replay them: the library enqueues kernels only (no allocation, no memset,
no host synchronisation), so the captured launches are the eager ones. The step number's
scalars are taken at capture, so every replay applies step `t` again to the evolving
weights and moments; the eager reference makes the same calls with the same `t`. Each
replay is checked against the eager state after as many applications, bit for bit, with
the host synchronising and reading back between replays. The allocation-free unfused
baseline is captured the same way (its dW lives in the library's static scratch).
"""
import numpy as np
import pytest
import torch

from oracle import optim
from synth import LayerSpec, draw_layer_batch, draw_layer_init
from tests import _parity as P

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _forge():
    import optimizer_gemm_amd as f
    return f


def _gh(hp):
    return dict(hp, nesterov=int(bool(hp["nesterov"])), stochastic_round=1)


def _state(f, W0, opt, fmt):
    W = P.dev_bf16(W0)
    m, v, ms, vs = f.new_states(W, opt, fmt)
    return W, m, v, ms, vs


def _snap(ts):
    return [None if t is None else P.host(t).copy() for t in ts]


@pytest.mark.parametrize("fmt", ["f32", "q8"])
def test_captured_layer_step_replays_equal_eager(fmt):
    f = _forge()
    specs = [LayerSpec("g1", 512, 768, 256), LayerSpec("g2", 1024, 512, 256)]
    opt, t = "adamw", 5
    hp = _gh(optim.hyper(opt))
    layers = []
    for li, spec in enumerate(specs):
        X, dY = draw_layer_batch(150, li, 1, spec)
        layers.append(dict(spec=spec, X=P.dev_bf16(X), dY=P.dev_bf16(dY), W0=draw_layer_init(150, li, spec),
                           seed=0xC0FFEE ^ li))
    code = "linear"

    def step(st, dX):
        for k, L in enumerate(layers):
            W, m, v, ms, vs = st[k]
            f.dgrad(L["dY"], W, dX[k])
            f.wgrad_step(L["X"], L["dY"], W, m, v, opt, hp, t, L["seed"], ms, vs, code=code)

    # eager: REPLAYS applications, a snapshot after each
    eager = [_state(f, L["W0"], opt, fmt) for L in layers]
    dX_e = [torch.empty((L["spec"].T, L["spec"].inn), dtype=torch.bfloat16, device="cuda") for L in layers]
    ref = []
    for _ in range(REPLAYS):
        step(eager, dX_e)
        torch.cuda.synchronize()
        ref.append([_snap(list(st) + [dX_e[k]]) for k, st in enumerate(eager)])

    # captured once, replayed
    cap = [_state(f, L["W0"], opt, fmt) for L in layers]
    dX_g = [torch.empty_like(d) for d in dX_e]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cap, dX_g)
    torch.cuda.synchronize()
    print(f"[case] graph of {2 * len(layers)} launches, {fmt} moments", flush=True)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        got = [_snap(list(st) + [dX_g[k]]) for k, st in enumerate(cap)]
        for k in range(len(layers)):
            for name, a, b in zip(("W", "m", "v", "m_scale", "v_scale", "dX"), got[k], ref[r][k]):
                if a is None:
                    assert b is None
                    continue
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {r}, layer {k}: {name} differs"
        print(f"[ok] replay {r}: every tensor equals the eager state after {r + 1} applications", flush=True)
    del g


def test_captured_noalloc_baseline_replays_equal_eager():
    f = _forge()
    spec = LayerSpec("gn", 640, 1024, 200)
    opt, t, seed = "nadam", 3, 77
    hp = _gh(optim.hyper(opt))
    X, dY = draw_layer_batch(151, 0, 1, spec)
    Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
    W0 = draw_layer_init(151, 0, spec)
    eager = _state(f, W0, opt, "f32")
    ref = []
    for _ in range(REPLAYS):
        f.wgrad_unfused_noalloc(Xd, dYd, *eager[:3], opt, hp, t, seed)
        torch.cuda.synchronize()
        ref.append(_snap(eager[:3]))
    cap = _state(f, W0, opt, "f32")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f.wgrad_unfused_noalloc(Xd, dYd, *cap[:3], opt, hp, t, seed)
    torch.cuda.synchronize()
    # (the capture itself may take a little of torch's memory; the replays take none)
    base = torch.cuda.memory_allocated()
    print("[case] graph of the allocation-free unfused baseline", flush=True)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("W", "m", "v"), _snap(cap[:3]), ref[r]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {r}: {name} differs"
    assert torch.cuda.memory_allocated() == base
    del g


def test_captured_grouped_step_replays_equal_eager():
    """The grouped fused step (three layers on one X) captured once and replayed, against
    the same call made eagerly, bit for bit after each replay."""
    f = _forge()
    specs = [LayerSpec("gq", 512, 768, 256), LayerSpec("gk", 128, 768, 256), LayerSpec("gv", 128, 768, 256)]
    opt, t = "adamw", 4
    hp = _gh(optim.hyper(opt))
    X, _ = draw_layer_batch(152, 0, 1, specs[0])
    Xd = P.dev_bf16(X)
    dYs = [P.dev_bf16(draw_layer_batch(152, k, 1, s)[1]) for k, s in enumerate(specs)]
    W0 = [draw_layer_init(152, k, s) for k, s in enumerate(specs)]
    seeds = [0xBEEF ^ k for k in range(len(specs))]

    def step(st):
        f.wgrad_step_group(Xd, dYs, [s[0] for s in st], [s[1] for s in st], [s[2] for s in st], opt, hp, t, seeds)

    eager = [_state(f, w, opt, "f32") for w in W0]
    ref = []
    for _ in range(REPLAYS):
        step(eager)
        torch.cuda.synchronize()
        ref.append([_snap(st[:3]) for st in eager])
    cap = [_state(f, w, opt, "f32") for w in W0]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cap)
    torch.cuda.synchronize()
    print("[case] graph of one grouped launch over 3 layers", flush=True)
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        for k, st in enumerate(cap):
            for name, a, b in zip(("W", "m", "v"), _snap(st[:3]), ref[r][k]):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {r}, layer {k}: {name} differs"
        print(f"[ok] replay {r}", flush=True)
    del g
