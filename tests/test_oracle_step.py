"""End-to-end pins for the oracle's fused step (no GPU).

Closed forms through the whole composition (gradient -> update -> storage), and
the pages' exactness claim: a tile-wise schedule gives the same step as the
full-gradient step for element-wise optimizers (§2 "Precision and fidelity").
"""
import os

import numpy as np
import pytest

from oracle import gemm, optim, q8, rounding, step
from synth import inputs

GOLDEN_SPLITMIX = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_published.txt")


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


# ---------------------------------------------------------------- bfloat16 moment states
def test_moment_bits_are_fields_of_the_published_words():
    # the m and v draws are bits 32..47 and 16..31 of the same SplitMix64 word as the
    # weight's: for counter c it is output number c+1 of the generator, checked against
    # the published outputs for seed 1234567 and the sequential generator
    lines = [l.split() for l in open(GOLDEN_SPLITMIX) if l.strip() and not l.startswith("#")]
    seed = int(lines[0][1])
    words = [int(l[0]) for l in lines[1:]]
    idx = np.arange(len(words), dtype=np.uint64)
    for s, shift in ((0, 48), (1, 32), (2, 16)):
        got = rounding.rand16(seed, 0, idx, stream=s)
        np.testing.assert_array_equal(got, np.array([(z >> shift) & 0xFFFF for z in words], dtype=np.uint32))
    seed = 0x0123456789ABCDEF
    seq = rounding.splitmix64_py(seed, 40)
    for s, shift in ((1, 32), (2, 16)):
        got = rounding.rand16(seed, 0, np.arange(40, dtype=np.uint64), stream=s)
        np.testing.assert_array_equal(got, np.array([(z >> shift) & 0xFFFF for z in seq], dtype=np.uint32))


def test_moment_streams_are_uncorrelated_with_the_weight_stream():
    idx = np.arange(200_000, dtype=np.uint64)
    r = [rounding.rand16(77, 3, idx, stream=s).astype(np.float64) for s in (0, 1, 2)]
    for a, b in ((0, 1), (0, 2), (1, 2)):
        assert abs(np.corrcoef(r[a], r[b])[0, 1]) < 0.01
        assert np.mean(r[a] == r[b]) < 1e-3


def test_bf16_moments_exact_when_representable():
    # integer-valued X and dY: g is an integer below 2^8, exact in bfloat16, so the
    # SGD-momentum buffer of step 1 (m = g) is stored exactly whatever the random bits
    rng = np.random.default_rng(5)
    X = rng.integers(-2, 3, size=(16, 64)).astype(np.float32)
    dY = rng.integers(-2, 3, size=(16, 8)).astype(np.float32)
    Xb, dYb = inputs.bf16_bits_from_f32(X), inputs.bf16_bits_from_f32(dY)
    W = inputs.bf16_bits_from_f32(np.zeros((8, 64), np.float32))
    m0 = inputs.bf16_bits_from_f32(np.zeros((8, 64), np.float32))
    hp = optim.hyper("sgd_momentum", weight_decay=0.0)
    g = dY.astype(np.float64).T @ X.astype(np.float64)
    for seed in (1, 2, 3):
        out = step.wgrad_step("sgd_momentum", Xb, dYb, W, m0, None, hp, 1, seed, state="bf16")
        np.testing.assert_array_equal(rounding.bf16_to_f64(out["m"]), g)


def test_bf16_moments_round_to_a_neighbour_and_are_unbiased():
    spec = inputs.LayerSpec("t", 8, 64, 32)
    W = inputs.draw_layer_init(9, 3, spec)
    X, dY = inputs.draw_layer_batch(9, 3, 1, spec)
    hp = optim.hyper("adamw")
    z = inputs.bf16_bits_from_f32(np.zeros(W.shape, np.float32))
    ref = step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, 0, state="f32")
    n = 2000
    acc = {"m": np.zeros(W.shape), "v": np.zeros(W.shape)}
    for s in range(n):
        out = step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, s, state="bf16")
        for k in acc:
            val = rounding.bf16_to_f64(out[k])
            x32 = ref[k].astype(np.float64)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x32), 1e-38))) - 7)
            assert np.all(np.abs(val - x32) < ulp)            # one of the two bfloat16 neighbours
            acc[k] += val
    for k in acc:
        x32 = ref[k].astype(np.float64)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x32), 1e-38))) - 7)
        assert np.max(np.abs(acc[k] / n - x32) / ulp) < 4.5 * 0.5 / np.sqrt(n) * 2
    # the weight update does not see the rounding of the moments
    np.testing.assert_array_equal(out["x32"], step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, s, state="f32")["x32"])


def test_bf16_moments_round_to_nearest_when_sr_is_off():
    spec = inputs.LayerSpec("t", 8, 64, 32)
    W = inputs.draw_layer_init(9, 4, spec)
    X, dY = inputs.draw_layer_batch(9, 4, 1, spec)
    hp = optim.hyper("adamw")
    z = inputs.bf16_bits_from_f32(np.zeros(W.shape, np.float32))
    ref = step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, 0, state="f32", sr=False)
    out = step.wgrad_step("adamw", X, dY, W, z, z, hp, 1, 0, state="bf16", sr=False)
    t = __import__("torch")
    for k in ("m", "v"):
        want = t.from_numpy(ref[k]).to(t.bfloat16).view(t.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(out[k], want)
