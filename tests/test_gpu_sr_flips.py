"""Stochastic-rounding flip rate of the fused step over several input seeds.

The bf16 weight path is bit-exact against the oracle except where the FP32 sum over the
tokens differs from the float64 one in a bit that decides the rounding: a differing
element flips its stochastic rounding with probability |dx32| / 2^16 (dx32 in float32
ulps). RMSprop's second step on the Qwen3-14B MLP weight (17408 x 5120, 4096 tokens) is
the most sensitive case of the sweep (its early updates are about ten learning rates,
half the weights' size). Per seed the test checks every flip (one step, explained), and
holds the count to the budget of what a model of the matrix instruction's FP32 summation
in the kernel's order predicts for the same inputs (flip_budget). The rate it reports,
about 0.011% over the eight seeds, is above the 0.01% that the bf16 weight path is
otherwise held to: at this step the flips the FP32 sum itself causes exceed that budget.
"""
import numpy as np
import pytest
import torch

from oracle import optim
from synth import WORKLOADS, draw_layer_batch, draw_layer_init, sample_rows
from tests import _parity as P

pytestmark = pytest.mark.gpu

SEEDS = 8


@pytest.mark.timeout(900)
def test_rmsprop_step_two_flip_rate_over_eight_seeds():
    import optimizer_gemm_amd as f
    wl = WORKLOADS["qwen14b_mlp_4096"]
    spec = wl.layers[0]
    opt = "rmsprop"
    hp = optim.hyper(opt)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    order_of = P.wgrad_tile_order(spec.out, spec.inn, cus)
    assert order_of is not None
    rows_total, flips, preds = 0, [], []
    for s in range(SEEDS):
        layer = 100 + s
        print(f"[case] rmsprop qwen mlp seed {s} (layer {layer})", flush=True)
        W0 = draw_layer_init(wl.config, layer, spec)
        sel = sample_rows(wl.config, layer, spec.out, 96)
        Wd = P.dev_bf16(W0)
        m, v, ms, vs = f.new_states(Wd, opt, "f32")
        seed = (0x5EED0000 + wl.config) ^ layer
        gh = dict(hp, nesterov=int(bool(hp["nesterov"])), stochastic_round=1)
        for t in (1, 2):
            X, dY = draw_layer_batch(wl.config, layer, t, spec)
            Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
            before = P.snapshot((Wd, m, v, ms, vs), sel) if t == 2 else None
            f.wgrad_step(Xd, dYd, Wd, m, v, opt, gh, t, seed, ms, vs)
            torch.cuda.synchronize()
            del Xd, dYd
        after = P.snapshot((Wd, m, v, ms, vs), sel)
        W_b, m_b, v_b, _, _ = before
        from oracle import step as ostep
        ref = ostep.wgrad_step(opt, X, dY, W_b, m_b, v_b, hp, 2, seed, rows=sel)
        ok, n, unexp, detail = P.bf16_step_explained(after[0], ref, opt, X, dY, W_b, m_b, v_b, hp, 2, seed, "bf16",
                                                     "f32", sel, frac=1.0)
        pred = P.predicted_flips(opt, X, dY, W_b, m_b, v_b, hp, 2, seed, "bf16", "f32", sel, None, None, None, ref,
                                 "W", True, order_of)
        print(f"[flips] seed {s}: {n} of {after[0].size} ({100 * n / after[0].size:.4f}%), predicted "
              f"{pred:.1f} (budget {P.flip_budget(pred)}), unexplained {unexp}", flush=True)
        assert unexp == 0, f"seed {s}: {unexp} differing weights not explained: {detail}"
        assert n <= P.flip_budget(pred), f"seed {s}: {n} flips, above the model's budget {P.flip_budget(pred)}"
        flips.append(n)
        preds.append(pred)
        rows_total += after[0].size
    rate = sum(flips) / rows_total
    print(f"[flips] rmsprop step 2 over {SEEDS} seeds: {sum(flips)} of {rows_total} = {100 * rate:.4f}% "
          f"(budget 0.0100%), predicted {sum(preds):.1f}", flush=True)
