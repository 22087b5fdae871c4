"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The GPU runs whole layers; the float64 oracle checks a seeded sample of output
rows (row-sampled mode: the same oracle restricted to those rows, exact because
the update is element-wise and INT8 blocks never cross rows). Every checked
step is teacher-forced from the GPU's previous state. dgrad is checked on a
seeded sample of token rows.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import gemm, optim
from synth import WORKLOADS, LayerSpec, draw_layer_batch, draw_layer_init, f32_from_bf16_bits, sample_rows
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _forge():
    import optimizer_gemm_amd as f
    return f


def _gh(hp, sr=True):
    return dict(hp, nesterov=int(bool(hp["nesterov"])), stochastic_round=int(sr))


def _check_dgrad(f, dYd, Wd, dY, W_bits, config, layer, n_tok=48):
    dX = f.dgrad(dYd, Wd)
    torch.cuda.synchronize()
    T = dY.shape[0]
    trows = np.sort(np.random.default_rng(config * 1000 + layer).choice(T, size=min(n_tok, T), replace=False))
    ref = f32_from_bf16_bits(dY[trows]).astype(np.float64) @ f32_from_bf16_bits(W_bits).astype(np.float64)
    bad, worst = P.dgrad_bf16_ok(P.host_bits(dX)[trows], ref)
    assert bad == 0, f"dgrad: {bad} sampled dX elements beyond one bf16 ulp (worst {worst:.3g})"


def _run_layer(f, wl, li, spec, opt, n_steps, check_steps, n_rows, check_dgrad_step=1):
    hp = optim.hyper(opt)
    seed = (0x5EED0000 + wl.config) ^ li
    W0 = draw_layer_init(wl.config, li, spec)
    Wd = P.dev_bf16(W0)
    m, v, ms, vs = f.new_states(Wd, opt, wl.state)
    sel = sample_rows(wl.config, li, spec.out, n_rows)
    for t in range(1, n_steps + 1):
        X, dY = draw_layer_batch(wl.config, li, t, spec)
        Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
        check = t in check_steps
        if t == check_dgrad_step:
            _check_dgrad(f, dYd, Wd, dY, P.host(Wd), wl.config, li)
        before = P.snapshot((Wd, m, v, ms, vs), sel) if check else None
        f.wgrad_step(Xd, dYd, Wd, m, v, opt, _gh(hp, wl.stochastic_round), t, seed, ms, vs,
                     code=P.state_code(wl.state))
        torch.cuda.synchronize()
        if check:
            after = P.snapshot((Wd, m, v, ms, vs), sel)
            P.verify_step(opt, X, dY, before, after, hp, t, seed, "bf16", wl.state, wl.stochastic_round, sel)
            print(f"[ok] {spec.name} {spec.out}x{spec.inn} T={spec.T} {opt} step {t}", flush=True)
        del Xd, dYd


@pytest.mark.timeout(300)
def test_q_proj_8192_ten_steps():
    f = _forge()
    wl = WORKLOADS["q_proj_8192"]
    _run_layer(f, wl, 0, wl.layers[0], "adamw", 10, set(range(1, 11)), 256)


@pytest.mark.timeout(300)
def test_q_proj_8192_whole_layer_first_step():
    # every one of the 16.8 M weights and moments of the q_proj layer against the oracle
    # (the full float64 dY^T X over 8192 tokens), not a sample of rows
    f = _forge()
    wl = WORKLOADS["q_proj_8192"]
    spec = wl.layers[0]
    _run_layer(f, wl, 1, spec, "adamw", 1, {1}, spec.out)


@pytest.mark.timeout(300)
def test_llama8b_decoder_layer_all_seven_linears():
    f = _forge()
    wl = WORKLOADS["llama8b_layer_8192"]
    for li, spec in enumerate(wl.layers):
        _run_layer(f, wl, li, spec, "adamw", 1, {1}, 128)


def test_llama8b_tp8_shards_all_seven_linears():
    # one GPU's 8-way tensor-parallel shards (k/v: 128 x 4096, 32 tiles of 128x128)
    f = _forge()
    wl = WORKLOADS["llama8b_tp8_8192"]
    for li, spec in enumerate(wl.layers):
        _run_layer(f, wl, li, spec, "adamw", 2, {1, 2}, 96)


@pytest.mark.timeout(600)
def test_down_proj_int8_states_twenty_steps():
    f = _forge()
    wl = WORKLOADS["down_q8_16384"]
    _run_layer(f, wl, 0, wl.layers[0], "adamw", 20, {1, 2, 3, 10, 20}, 128)


@pytest.mark.timeout(600)
def test_down_proj_dynamic_code_states_five_steps():
    f = _forge()
    wl = dataclasses.replace(WORKLOADS["down_q8_16384"], state="q8dyn")
    _run_layer(f, wl, 1, wl.layers[0], "adamw", 5, {1, 2, 5}, 96)


@pytest.mark.timeout(600)
def test_qwen14b_mlp_eight_optimizers_ten_steps():
    # all eight optimizers on the same per-step inputs; every step checked on sampled rows
    f = _forge()
    wl = WORKLOADS["qwen14b_mlp_4096"]
    spec = wl.layers[0]
    W0 = draw_layer_init(wl.config, 0, spec)
    sel = sample_rows(wl.config, 0, spec.out, 96)
    runs = {}
    for opt in wl.optimizers:
        Wd = P.dev_bf16(W0)
        runs[opt] = (Wd,) + tuple(f.new_states(Wd, opt, "f32"))
    for t in range(1, wl.steps + 1):
        X, dY = draw_layer_batch(wl.config, 0, t, spec)
        Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
        g = gemm.wgrad_rows(f32_from_bf16_bits(X), f32_from_bf16_bits(dY), sel)
        for opt in wl.optimizers:
            Wd, m, v, ms, vs = runs[opt]
            hp = optim.hyper(opt)
            seed = (0x5EED0000 + wl.config) ^ optim.OPTIMIZERS.index(opt)
            before = P.snapshot((Wd, m, v, ms, vs), sel)
            f.wgrad_step(Xd, dYd, Wd, m, v, opt, _gh(hp), t, seed, ms, vs)
            torch.cuda.synchronize()
            after = P.snapshot((Wd, m, v, ms, vs), sel)
            P.verify_step(opt, X, dY, before, after, hp, t, seed, "bf16", "f32", True, sel, g=g)
        print(f"[ok] qwen mlp step {t}: all eight optimizers", flush=True)
        del Xd, dYd


@pytest.mark.timeout(300)
def test_largest_weight_the_abi_accepts_int8_states_and_dgrad():
    # W 32760 x 32768 bf16 is 2,146,959,360 bytes, just below the 2^31-byte limit of a
    # tensor (all kernel addressing is 32-bit buffer offsets; rows stay multiples of 8
    # elements, and 32760 leaves a ragged last tile row): the fused AdamW step with
    # INT8 states is checked on sampled rows that include the last ones, and dgrad (which
    # reads all of W) on sampled tokens and columns, before the step as the method requires.
    f = _forge()
    out, inn, T = 32760, 32768, 64
    spec = LayerSpec("max", out, inn, T)
    print(f"[case] largest weight {out}x{inn} bf16 ({out * inn * 2} bytes), T={T}, AdamW + INT8 states",
          flush=True)
    g = torch.Generator(device="cuda").manual_seed(1234)
    Wd = (torch.randn(out, inn, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    m, v, ms, vs = f.new_states(Wd, "adamw", "q8")
    hp = optim.hyper("adamw")
    seed = 0x5EED_7777
    sel = np.unique(np.concatenate([sample_rows(77, 0, out, 24), [0, 1, out // 2, out - 2, out - 1]]))
    cols = np.unique(np.concatenate([np.random.default_rng(3).choice(inn, 24, replace=False), [0, inn - 1]]))
    for t in (1, 2):
        X, dY = draw_layer_batch(77, 0, t, spec)
        Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
        if t == 1:
            dX = f.dgrad(dYd, Wd)
            torch.cuda.synchronize()
            Wcols = P.host(Wd.index_select(1, torch.as_tensor(cols, device="cuda")))
            ref = f32_from_bf16_bits(dY).astype(np.float64) @ f32_from_bf16_bits(Wcols).astype(np.float64)
            bad, worst = P.dgrad_bf16_ok(P.host_bits(dX)[:, cols], ref)
            assert bad == 0, f"dgrad: {bad} sampled dX elements beyond one bf16 ulp (worst {worst:.3g})"
        before = P.snapshot((Wd, m, v, ms, vs), sel)
        f.wgrad_step(Xd, dYd, Wd, m, v, "adamw", _gh(hp), t, seed, ms, vs)
        torch.cuda.synchronize()
        after = P.snapshot((Wd, m, v, ms, vs), sel)
        P.verify_step("adamw", X, dY, before, after, hp, t, seed, "bf16", "q8", True, sel)
        print(f"[ok] largest weight, step {t}", flush=True)
    del Wd, m, v, ms, vs
