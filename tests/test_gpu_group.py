"""The grouped fused step (layers that share X in one launch) against the oracle, through the C ABI.

Each layer of a group is checked with the same teacher-forced oracle step as a layer of its
own (tests/_parity.py): its element indices and random streams are its own, only the tile
shape (the order of the FP32 summation over tokens) is chosen for the group. A group of one
layer, on a shape whose tiles the group and the single-layer launcher choose alike, equals
the single-layer call bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import optim
from synth import LayerSpec, draw_layer_batch, draw_layer_batch_fp8, draw_layer_init, sample_rows
from tests import _parity as P
from tests.test_gpu_fp8 import dev_fp8, dev_scale

pytestmark = pytest.mark.gpu


def _forge():
    import optimizer_gemm_amd as f
    return f


def _gh(hp):
    return dict(hp, nesterov=int(bool(hp["nesterov"])), stochastic_round=1)


def _run_group(outs, inn, T, opt, state, cfg, steps=2, n_rows=None):
    """Steps 1..steps of a group of len(outs) layers on one X, each checked on (sampled) rows."""
    f = _forge()
    hp = optim.hyper(opt)
    code = "dynamic" if state == "q8dyn" else "linear"
    specs = [LayerSpec(f"g{k}", out, inn, T) for k, out in enumerate(outs)]
    seeds = [(0x6A0000 + cfg) ^ k for k in range(len(outs))]
    # a layer with no rows (out = 0) is built directly: it takes part in the call only
    init = lambda k, s: draw_layer_init(cfg, k, s) if s.out else np.zeros((0, inn), np.uint16)  # noqa: E731
    Ws = [P.dev_bf16(init(k, s)) for k, s in enumerate(specs)]
    st = [f.new_states(W, opt, state) for W in Ws]
    rows = [np.arange(s.out) if n_rows is None or s.out <= n_rows else sample_rows(cfg, k, s.out, n_rows)
            for k, s in enumerate(specs)]
    print(f"[case] group {outs} x {inn}, T={T}, {opt}, {state} moments", flush=True)
    for t in range(1, steps + 1):
        X, _ = draw_layer_batch(cfg, 0, t, specs[0])
        dYs = [draw_layer_batch(cfg, k, t, s)[1] if s.out else np.zeros((T, 0), np.uint16) for k, s in enumerate(specs)]
        Xd = P.dev_bf16(X)
        dYd = [P.dev_bf16(d) for d in dYs]
        before = [P.snapshot((W, *s), r) if W.shape[0] else None for W, s, r in zip(Ws, st, rows)]
        f.wgrad_step_group(Xd, dYd, Ws, [s[0] for s in st], [s[1] for s in st], opt, _gh(hp), t, seeds,
                           [s[2] for s in st], [s[3] for s in st], code=code)
        torch.cuda.synchronize()
        for k, spec in enumerate(specs):
            if spec.out == 0:
                continue
            after = P.snapshot((Ws[k], *st[k]), rows[k])
            P.verify_step(opt, X, dYs[k], before[k], after, hp, t, seeds[k], "bf16", state, True, rows[k])
        print(f"[ok] step {t}: every layer of the group", flush=True)


@pytest.mark.parametrize("state", ["f32", "bf16", "q8", "q8dyn"])
def test_group_ragged_layers(state):
    # three layers of one input (q, k, v-like, the second ragged), 520 tokens (ragged stages)
    _run_group((384, 136, 128), 1024, 520, "adamw", state, cfg=160)


@pytest.mark.parametrize("opt", ["sgd", "sgd_momentum", "lion", "rmsprop", "adagrad", "nadam", "radam"])
def test_group_every_optimizer(opt):
    _run_group((256, 192), 512, 200, opt, "f32", cfg=161)


def test_group_large_tiles_four_layers():
    # enough tiles for the 256x256 configuration across the four layers (a ragged last one)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    outs = (1024, 256, 256, 520)
    assert 2 * 16 * sum(-(-o // 256) for o in outs) > cus
    _run_group(outs, 4096, 300, "adamw", "f32", cfg=162, steps=1, n_rows=48)


def test_group_with_empty_layer_and_zero_tokens():
    _run_group((256, 0, 128), 512, 0, "adamw", "f32", cfg=163, steps=1)


def test_group_of_one_equals_single_layer_call():
    f = _forge()
    spec = LayerSpec("g", 512, 768, 256)
    hp = _gh(optim.hyper("adamw"))
    X, dY = draw_layer_batch(164, 0, 1, spec)
    Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
    W0 = draw_layer_init(164, 0, spec)
    outs = []
    for grouped in (False, True):
        W = P.dev_bf16(W0)
        m, v, _, _ = f.new_states(W, "adamw", "f32")
        for t in (1, 2):
            if grouped:
                f.wgrad_step_group(Xd, [dYd], [W], [m], [v], "adamw", hp, t, [99])
            else:
                f.wgrad_step(Xd, dYd, W, m, v, "adamw", hp, t, 99)
        torch.cuda.synchronize()
        outs.append([P.host(x).copy() for x in (W, m, v)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("state", ["f32", "q8"])
def test_group_band_split_attention_projections(state):
    # q, k, v of a Llama-3.1-8B layer: 384 large tiles, a half-full last round on 256 CUs;
    # there q runs as one round of large tiles and k, v as one round of band tiles
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[case] {cus} compute units", flush=True)
    _run_group((4096, 1024, 1024), 4096, 300, "adamw", state, cfg=165, steps=1, n_rows=48)


def _run_group_fp8(outs, inn, T, opt, state, cfg, dy_fmt="e5m2", steps=2, n_rows=None):
    """As _run_group with FP8 inputs: X (E4M3, layer 0's draw) shared, each layer's dY in
    dy_fmt with its own scale; each layer checked with the FP8 gradient bound."""
    f = _forge()
    hp = optim.hyper(opt)
    specs = [LayerSpec(f"g{k}", out, inn, T) for k, out in enumerate(outs)]
    seeds = [(0x6B0000 + cfg) ^ k for k in range(len(outs))]
    Ws = [P.dev_bf16(draw_layer_init(cfg, k, s)) for k, s in enumerate(specs)]
    st = [f.new_states(W, opt, state) for W in Ws]
    rows = [np.arange(s.out) if n_rows is None or s.out <= n_rows else sample_rows(cfg, k, s.out, n_rows)
            for k, s in enumerate(specs)]
    print(f"[case] fp8 group {outs} x {inn}, T={T}, dY {dy_fmt}, {opt}, {state} moments", flush=True)
    for t in range(1, steps + 1):
        draws = [draw_layer_batch_fp8(cfg, k, t, s, "e4m3", dy_fmt) for k, s in enumerate(specs)]
        Xq, sx = draws[0][0], draws[0][2]
        before = [P.snapshot((W, *s), r) for W, s, r in zip(Ws, st, rows)]
        f.wgrad_step_group(dev_fp8(Xq, "e4m3"), [dev_fp8(d[1], dy_fmt) for d in draws], Ws, [s[0] for s in st],
                           [s[1] for s in st], opt, _gh(hp), t, seeds, [s[2] for s in st], [s[3] for s in st],
                           code=P.state_code(state), x_scale=dev_scale(sx), dy_scales=[dev_scale(d[3]) for d in draws])
        torch.cuda.synchronize()
        for k in range(len(specs)):
            after = P.snapshot((Ws[k], *st[k]), rows[k])
            P.verify_step(opt, Xq, draws[k][1], before[k], after, hp, t, seeds[k], "bf16", state, True, rows[k],
                          fp8=("e4m3", dy_fmt, sx, draws[k][3]))
        print(f"[ok] step {t}: every layer of the FP8 group", flush=True)


@pytest.mark.parametrize("state", ["f32", "q8"])
def test_group_fp8_ragged_layers(state):
    # FP8 rows are multiples of 16 bytes: 144 = 128 + 16 output rows, 520 = 8 * 64 + 8 tokens
    _run_group_fp8((384, 144, 128), 1024, 520, "adamw", state, cfg=170)


def test_group_fp8_large_tiles_e4m3_gradients():
    # 160 tiles of 256x256 over four layers: more than half a round, so the large FP8 tiles
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    outs = (1024, 512, 512, 512)
    assert 2 * 16 * sum(o // 256 for o in outs) > cus
    _run_group_fp8(outs, 4096, 300, "adamw", "f32", cfg=171, dy_fmt="e4m3", steps=1, n_rows=48)


def test_group_fp8_of_one_equals_single_layer_call():
    f = _forge()
    spec = LayerSpec("g", 512, 768, 256)
    hp = _gh(optim.hyper("adamw"))
    Xq, dYq, sx, sd = draw_layer_batch_fp8(172, 0, 1, spec, "e4m3", "e5m2")
    Xd, dYd, xs, ds = dev_fp8(Xq, "e4m3"), dev_fp8(dYq, "e5m2"), dev_scale(sx), dev_scale(sd)
    W0 = draw_layer_init(172, 0, spec)
    outs = []
    for grouped in (False, True):
        W = P.dev_bf16(W0)
        m, v, _, _ = f.new_states(W, "adamw", "f32")
        for t in (1, 2):
            if grouped:
                f.wgrad_step_group(Xd, [dYd], [W], [m], [v], "adamw", hp, t, [99], x_scale=xs, dy_scales=[ds])
            else:
                f.wgrad_step(Xd, dYd, W, m, v, "adamw", hp, t, 99, x_scale=xs, dy_scale=ds)
        torch.cuda.synchronize()
        outs.append([P.host(x).copy() for x in (W, m, v)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_group_members_with_row_pitch():
    # members whose dY, W and moments are views into wider buffers (row pitch > columns):
    # each member's pitches travel in its own table entry
    f = _forge()
    hp = optim.hyper("adamw")
    outs, inn, T, cfg = (256, 136), 512, 200, 173
    specs = [LayerSpec(f"p{k}", out, inn, T) for k, out in enumerate(outs)]
    seeds = [0x7100 ^ k for k in range(2)]
    X, _ = draw_layer_batch(cfg, 0, 1, specs[0])
    dYs = [draw_layer_batch(cfg, k, 1, s)[1] for k, s in enumerate(specs)]
    W0 = [draw_layer_init(cfg, k, s) for k, s in enumerate(specs)]
    pad = (64, 128)

    def pitched(a, p, dtype):
        base = torch.zeros((a.shape[0], a.shape[1] + p), dtype=dtype, device="cuda")
        v = base[:, :a.shape[1]]
        v.copy_(a)
        return v

    dY_d = [pitched(P.dev_bf16(d), p, torch.bfloat16) for d, p in zip(dYs, pad)]
    Ws = [pitched(P.dev_bf16(w), p, torch.bfloat16) for w, p in zip(W0, pad)]
    ms = [pitched(torch.zeros(w.shape, device="cuda"), p, torch.float32) for w, p in zip(W0, pad)]
    vs = [pitched(torch.zeros(w.shape, device="cuda"), p, torch.float32) for w, p in zip(W0, pad)]
    assert all(w.stride(0) != w.shape[1] for w in Ws)
    print("[case] group of 2 with pitched dY, W, m, v", flush=True)
    rows = [np.arange(s.out) for s in specs]
    before = [P.snapshot((W, m, v, None, None), r) for W, m, v, r in zip(Ws, ms, vs, rows)]
    f.wgrad_step_group(P.dev_bf16(X), dY_d, Ws, ms, vs, "adamw", _gh(hp), 1, seeds)
    torch.cuda.synchronize()
    for k in range(2):
        after = P.snapshot((Ws[k], ms[k], vs[k], None, None), rows[k])
        P.verify_step("adamw", X, dYs[k], before[k], after, hp, 1, seeds[k], "bf16", "f32", True, rows[k])
    print("[ok] both members", flush=True)
