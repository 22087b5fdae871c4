"""Pins for the oracle's INT8 block-64 moment codec (no GPU).

The pages state block 64 (vs 2048 in standard 8-bit optimizers) to minimise
quantisation error (§2 "Precision and fidelity"); the oracle reads it as linear
absmax codes (signed /127 for m, unsigned /255 on sqrt(v) for v).
"""
import numpy as np
import pytest

from oracle import q8


def test_signed_absmax_maps_to_127_and_error_bound():
    rng = np.random.default_rng(0)
    m = rng.standard_normal((6, 256)) * 1e-3
    q, s = q8.quant_signed(m)
    assert q.dtype == np.int8 and s.shape == (6, 4) and s.dtype == np.float32
    blocks = m.reshape(6, 4, 64)
    qb = q.reshape(6, 4, 64)
    amax_pos = np.argmax(np.abs(blocks), axis=-1)
    picked = np.take_along_axis(qb, amax_pos[..., None], axis=-1)[..., 0]
    np.testing.assert_array_equal(np.abs(picked), 127)
    err = np.abs(q8.dequant_signed(q, s) - m).reshape(6, 4, 64)
    assert np.all(err <= s.astype(np.float64)[..., None] * (0.5 + 1e-6))


def test_sqrt_unsigned_absmax_maps_to_255_and_error_bound():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((3, 128)) * 1e-3) ** 2
    q, s = q8.quant_sqrt_unsigned(v)
    assert q.dtype == np.uint8
    rb = np.sqrt(v).reshape(3, 2, 64)
    pos = np.argmax(rb, axis=-1)
    np.testing.assert_array_equal(np.take_along_axis(q.reshape(3, 2, 64), pos[..., None], -1), 255)
    r_hat = np.sqrt(q8.dequant_sqrt_unsigned(q, s)).reshape(3, 2, 64)
    assert np.all(np.abs(r_hat - rb) <= s.astype(np.float64)[..., None] * (0.5 + 1e-6))


def test_zero_block():
    m = np.zeros((2, 128))
    m[1, 64:] = np.linspace(-1, 1, 64)
    q, s = q8.quant_signed(m)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] > 0
    assert np.all(q[0] == 0) and np.all(q[1, :64] == 0)
    assert np.all(q8.dequant_signed(q, s)[0] == 0)
    qv, sv = q8.quant_sqrt_unsigned(np.zeros((1, 64)))
    assert sv[0, 0] == 0 and np.all(qv == 0)


def test_block64_error_below_block2048():
    # the pages' reason for the small block: lower quantisation error, most visibly with outliers
    rng = np.random.default_rng(2)
    m = rng.standard_normal((8, 4096)) * 1e-3
    m[:, rng.integers(0, 4096, 40)] *= 100.0
    e64 = np.mean((q8.dequant_signed(*q8.quant_signed(m, 64), 64) - m) ** 2)
    e2048 = np.mean((q8.dequant_signed(*q8.quant_signed(m, 2048), 2048) - m) ** 2)
    assert e64 < 0.5 * e2048
    # without outliers the smaller block is still more accurate
    g = rng.standard_normal((8, 4096)) * 1e-3
    assert np.mean((q8.dequant_signed(*q8.quant_signed(g, 64), 64) - g) ** 2) < \
        np.mean((q8.dequant_signed(*q8.quant_signed(g, 2048), 2048) - g) ** 2)


def test_sqrt_code_keeps_v_nonzero_where_m_nonzero():
    # first AdamW step on Gaussian gradients: v = (1-b2) g^2, m = (1-b1) g
    rng = np.random.default_rng(3)
    g = rng.standard_normal((256, 1024))
    mq, ms = q8.quant_signed(0.1 * g)
    vq, vs = q8.quant_sqrt_unsigned(1e-3 * g * g)
    m_hat = q8.dequant_signed(mq, ms)
    v_hat = q8.dequant_sqrt_unsigned(vq, vs)
    assert np.mean((v_hat == 0) & (m_hat != 0)) == 0.0


def test_rejects_ragged_rows():
    with pytest.raises(ValueError):
        q8.quant_signed(np.zeros((2, 100)))
