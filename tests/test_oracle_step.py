"""End-to-end pins for the oracle's fused step (no GPU).

Closed forms through the whole composition (gradient -> update -> storage), and
the pages' exactness claim: a tile-wise schedule gives the same step as the
full-gradient step for element-wise optimizers (§2 "Precision and fidelity").
"""
import numpy as np
import pytest

from oracle import gemm, optim, q8, rounding, step
from synth import inputs


def _f32_layer(seed, T=64, n_out=32, n_in=48):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, n_in)).astype(np.float32)
    dY = (rng.standard_normal((T, n_out)) * 1e-2).astype(np.float32)
    W = (rng.standard_normal((n_out, n_in)) * 0.02).astype(np.float32)
    return X, dY, W


def test_sgd_step_is_w_minus_lr_dw():
    X, dY, W = _f32_layer(0)
    hp = optim.hyper("sgd", lr=0.05)
    out = step.wgrad_step("sgd", X, dY, W, None, None, hp, 1, 0, io="f32", sr=False)
    dW = dY.astype(np.float64).T @ X.astype(np.float64)
    np.testing.assert_array_equal(out["W"], (W.astype(np.float64) - 0.05 * dW).astype(np.float32))
    assert out["m"] is None and out["v"] is None


def test_adamw_first_step_sign_plus_decay():
    X, dY, W = _f32_layer(1)
    hp = optim.hyper("adamw")
    z = np.zeros_like(W)
    out = step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, 0, io="f32", sr=False)
    g = out["g"]
    expect = W.astype(np.float64) * (1 - 1e-3 * 0.01) - 1e-3 * g / (np.abs(g) + 1e-8)
    np.testing.assert_allclose(out["W"], expect.astype(np.float32), rtol=0, atol=1e-9)
    np.testing.assert_allclose(out["m"], (0.1 * g).astype(np.float32), rtol=1e-7)
    np.testing.assert_allclose(out["v"], (0.001 * g * g).astype(np.float32), rtol=1e-7)


@pytest.mark.parametrize("opt", optim.OPTIMIZERS)
def test_tilewise_schedule_equals_full_step(opt):
    # the same update applied per 128x128 tile with the tile's own gradient
    X, dY, W = _f32_layer(2, T=300, n_out=256, n_in=384)
    hp = optim.hyper(opt, weight_decay=0.01)
    slots = optim.SLOTS[opt]
    rng = np.random.default_rng(5)
    m = (rng.standard_normal(W.shape) * 1e-3) if "m" in slots else None
    v = (rng.standard_normal(W.shape) * 1e-3) ** 2 if "v" in slots else None
    full = optim.update(opt, W.astype(np.float64), gemm.wgrad(X, dY), m, v, hp, 4)
    theta = np.empty(W.shape)
    for o0 in range(0, 256, 128):
        for i0 in range(0, 384, 128):
            sl = (slice(o0, o0 + 128), slice(i0, i0 + 128))
            gt = np.zeros((128, 128))
            for t0 in range(0, 300, 64):
                gt += dY[t0:t0 + 64, sl[0]].astype(np.float64).T @ X[t0:t0 + 64, sl[1]].astype(np.float64)
            res = optim.update(opt, W[sl].astype(np.float64), gt,
                               None if m is None else m[sl], None if v is None else v[sl], hp, 4)
            theta[sl] = res[0]
    np.testing.assert_allclose(theta, full[0], rtol=1e-12, atol=1e-15)


def test_row_sampled_equals_full_rows_bf16_sr():
    spec = inputs.LayerSpec("t", 96, 128, 80)
    W = inputs.draw_layer_init(9, 0, spec)
    X, dY = inputs.draw_layer_batch(9, 0, 1, spec)
    hp = optim.hyper("adamw")
    m = np.zeros(W.shape, np.float32)
    full = step.wgrad_step("adamw", X, dY, W, m, m, hp, 1, 77)
    rows = np.array([1, 50, 95])
    part = step.wgrad_step("adamw", X, dY, W[rows], m[rows], m[rows], hp, 1, 77, rows=rows)
    np.testing.assert_array_equal(part["W"], full["W"][rows])
    np.testing.assert_array_equal(part["m"], full["m"][rows])


def test_bf16_sr_uses_row_major_index_and_step():
    spec = inputs.LayerSpec("t", 4, 64, 16)
    W = inputs.draw_layer_init(9, 1, spec)
    X, dY = inputs.draw_layer_batch(9, 1, 1, spec)
    hp = optim.hyper("sgd", lr=1e-2)
    out = step.wgrad_step("sgd", X, dY, W, None, None, hp, 5, 1234)
    r16 = rounding.rand16(1234, 5, np.arange(4 * 64, dtype=np.uint64)).reshape(4, 64)
    np.testing.assert_array_equal(out["W"], rounding.sr_bf16(out["x32"], r16))


def test_bf16_sr_step_is_unbiased_over_seeds():
    # the mean of the stored weight over many seeds approaches the float32 result
    spec = inputs.LayerSpec("t", 8, 64, 32)
    W = inputs.draw_layer_init(9, 2, spec)
    X, dY = inputs.draw_layer_batch(9, 2, 1, spec)
    hp = optim.hyper("sgd", lr=3e-3)
    acc = np.zeros((8, 64))
    n = 2000
    for s in range(n):
        acc += rounding.bf16_to_f64(step.wgrad_step("sgd", X, dY, W, None, None, hp, 1, s)["W"])
    x32 = step.wgrad_step("sgd", X, dY, W, None, None, hp, 1, 0)["x32"].astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x32))) - 7)
    assert np.max(np.abs(acc / n - x32) / ulp) < 4.5 * 0.5 / np.sqrt(n) * 2


def test_q8_state_step_updates_with_unquantised_moments():
    X, dY, W = _f32_layer(3, n_in=128)
    hp = optim.hyper("adamw")
    rng = np.random.default_rng(4)
    m0 = rng.standard_normal(W.shape) * 1e-3
    v0 = (rng.standard_normal(W.shape) * 1e-3) ** 2
    mq, ms = q8.quant_signed(m0)
    vq, vs = q8.quant_sqrt_unsigned(v0)
    out = step.wgrad_step("adamw", X, dY, W, mq, vq, hp, 3, 0, io="f32", state="q8", sr=False,
                          m_scale=ms, v_scale=vs)
    th, mn, vn = optim.update("adamw", W.astype(np.float64), out["g"], q8.dequant_signed(mq, ms),
                              q8.dequant_sqrt_unsigned(vq, vs), hp, 3)
    np.testing.assert_array_equal(out["W"], th.astype(np.float32))
    q_m, s_m = q8.quant_signed(mn)
    np.testing.assert_array_equal(out["m"], q_m)
    np.testing.assert_array_equal(out["m_scale"], s_m)
    assert out["v"].dtype == np.uint8 and out["v_scale"].shape == (32, 2)
