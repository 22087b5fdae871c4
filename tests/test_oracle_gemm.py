"""Pins for the oracle's weight and input gradients (no GPU).

The definition (FORGE explainer, §2 Method, core mechanism): dW[o,i] is the sum
over tokens of dY[t,o]*X[t,i]; dX = dY W uses the old weight (§5 limitations).
"""
import math

import numpy as np
import pytest

from oracle import gemm


def _bf16_like(rng, shape, scale=1.0):
    # values with 8 significant bits, so every product is exact in float64
    x = rng.standard_normal(shape) * scale
    e = np.floor(np.log2(np.abs(x) + 1e-300))
    return np.round(x / 2.0 ** (e - 7)) * 2.0 ** (e - 7)


def test_wgrad_brute_force_8x8():
    rng = np.random.default_rng(1)
    T, n_out, n_in = 8, 8, 8
    X = _bf16_like(rng, (T, n_in))
    dY = _bf16_like(rng, (T, n_out), 1e-2)
    ref = np.empty((n_out, n_in))
    for o in range(n_out):
        for i in range(n_in):
            ref[o, i] = math.fsum(dY[t, o] * X[t, i] for t in range(T))
    got = gemm.wgrad(X, dY)
    assert got.shape == (n_out, n_in)
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=1e-300)


def test_wgrad_rectangular_brute_force_catches_transpose():
    rng = np.random.default_rng(2)
    T, n_out, n_in = 5, 3, 7
    X = _bf16_like(rng, (T, n_in))
    dY = _bf16_like(rng, (T, n_out))
    got = gemm.wgrad(X, dY)
    assert got.shape == (n_out, n_in)
    for o in range(n_out):
        for i in range(n_in):
            assert got[o, i] == pytest.approx(math.fsum(dY[t, o] * X[t, i] for t in range(T)), rel=1e-15)


def test_wgrad_one_hot_closed_form():
    # X rows one-hot at column sel[t]  =>  dW[:, i] = sum of dY rows with sel[t] == i
    rng = np.random.default_rng(3)
    T, n_out, n_in = 40, 6, 9
    sel = rng.integers(0, n_in, size=T)
    X = np.zeros((T, n_in))
    X[np.arange(T), sel] = 1.0
    dY = rng.standard_normal((T, n_out))
    got = gemm.wgrad(X, dY)
    for i in range(n_in):
        np.testing.assert_allclose(got[:, i], dY[sel == i].sum(axis=0), rtol=1e-14, atol=1e-14)


def test_wgrad_ones_gives_column_sums():
    rng = np.random.default_rng(4)
    X = np.ones((17, 5))
    dY = rng.integers(-50, 50, size=(17, 4)).astype(np.float64)
    got = gemm.wgrad(X, dY)
    np.testing.assert_array_equal(got, np.repeat(dY.sum(axis=0)[:, None], 5, axis=1))


def test_wgrad_small_integers_exact():
    rng = np.random.default_rng(5)
    X = rng.integers(-8, 8, size=(33, 12)).astype(np.float64)
    dY = rng.integers(-8, 8, size=(33, 10)).astype(np.float64)
    ref = np.array([[sum(int(dY[t, o]) * int(X[t, i]) for t in range(33)) for i in range(12)] for o in range(10)])
    np.testing.assert_array_equal(gemm.wgrad(X, dY), ref)


def test_wgrad_rows_is_subset():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((50, 30))
    dY = rng.standard_normal((50, 20))
    rows = np.array([0, 3, 19])
    np.testing.assert_array_equal(gemm.wgrad_rows(X, dY, rows), gemm.wgrad(X, dY)[rows])


@pytest.mark.parametrize("shape", [(130, 300, 200), (64, 128, 128), (257, 129, 385)])
def test_tiled_equals_full(shape):
    # exactness claim: tile-wise accumulation equals the full gradient up to summation order
    T, n_out, n_in = shape
    rng = np.random.default_rng(7)
    X = rng.standard_normal((T, n_in))
    dY = rng.standard_normal((T, n_out))
    full = gemm.wgrad(X, dY)
    tiled = gemm.wgrad_tiled(X, dY, 128, 128, 64)
    scale = np.sqrt(T)
    assert np.max(np.abs(full - tiled)) <= 1e-12 * scale


def test_dgrad_brute_force():
    rng = np.random.default_rng(8)
    T, n_out, n_in = 8, 6, 7
    dY = _bf16_like(rng, (T, n_out))
    W = _bf16_like(rng, (n_out, n_in), 0.02)
    got = gemm.dgrad(dY, W)
    assert got.shape == (T, n_in)
    for t in range(T):
        for i in range(n_in):
            assert got[t, i] == pytest.approx(math.fsum(dY[t, o] * W[o, i] for o in range(n_out)), rel=1e-15)


def test_shape_errors():
    with pytest.raises(ValueError):
        gemm.wgrad(np.zeros((3, 4)), np.zeros((5, 4)))
    with pytest.raises(ValueError):
        gemm.dgrad(np.zeros((3, 4)), np.zeros((5, 4)))
