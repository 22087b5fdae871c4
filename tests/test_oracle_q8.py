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


# ---------------------------------------------------------------- dynamic 8-bit code
def test_dyn_tables_decades_and_endpoints():
    """Decade structure of the dynamic code: every decade [10^-(E+1), 10^-E] holds
    2^(n-1-E) codes, the largest of which is 10^-E; 0 and 1 are exact."""
    for table, n in ((q8.DYN_SIGNED, 7), (q8.DYN_UNSIGNED, 8)):
        assert table.dtype == np.float32 and table.size == 2 ** n
        assert table[0] == 0.0 and table[-1] == 1.0
        assert np.all(np.diff(table.astype(np.float64)) > 0)
        for E in range(n):
            lo, hi = 10.0 ** -(E + 1), 10.0 ** -E
            inside = table[(table > np.float32(lo) * (1 + 1e-6)) & (table <= np.float32(hi) * (1 + 1e-6))]
            assert inside.size == 2 ** (n - 1 - E), (n, E, inside.size)
            assert inside.max() == np.float32(hi)
        assert table[1] == np.float32(10.0 ** -(n - 1))
        # within a decade the codes are equally spaced (linear fraction)
        top = table[2 ** (n - 1):].astype(np.float64)
        np.testing.assert_allclose(np.diff(top), 0.9 / 2 ** (n - 1), rtol=0, atol=2 ** -22)


def test_dyn_encode_is_brute_force_nearest():
    """Encoding = the nearest table value, found by brute force over all codes."""
    rng = np.random.default_rng(5)
    for signed in (True, False):
        table = (q8.DYN_SIGNED if signed else q8.DYN_UNSIGNED).astype(np.float64)
        y = np.concatenate([rng.uniform(0, 1, 4000), 10.0 ** rng.uniform(-9, 0, 4000)])
        x = np.concatenate([[1.0], y]).reshape(-1, 1) * np.ones((1, 64))
        x[:, 0] = 1.0  # block absmax 1: y is the normalised value itself
        x[:, 1] = np.concatenate([[1.0], y]) * (-1 if signed else 1)
        q, s = (q8.quant_dyn_signed if signed else q8.quant_dyn_unsigned)(x)
        assert np.all(s == 1.0)
        k = (q[:, 1] & 0x7F) if signed else q[:, 1]
        a = np.abs(x[:, 1]).astype(np.float32).astype(np.float64)
        d = np.abs(a[:, None] - table[None, :])
        best = d.min(axis=1)
        assert np.all(d[np.arange(len(a)), k] == best), "not the nearest code"
        if signed:
            neg = x[:, 1] < 0
            assert np.all((q[:, 1] >= 0x80) == (neg & (k > 0)))


def test_dyn_codes_round_trip_and_absmax_exact():
    for signed, table in ((True, q8.DYN_SIGNED), (False, q8.DYN_UNSIGNED)):
        vals = table.astype(np.float64)
        x = np.zeros((vals.size, 64))
        x[:, 0] = 1.0
        x[:, 1] = -vals if signed else vals
        q, s = (q8.quant_dyn_signed if signed else q8.quant_dyn_unsigned)(x)
        k = (q[:, 1] & 0x7F) if signed else q[:, 1]
        np.testing.assert_array_equal(k, np.arange(vals.size))
        deq = (q8.dequant_dyn_signed if signed else q8.dequant_dyn_unsigned)(q, s)
        np.testing.assert_array_equal(deq[:, 1], x[:, 1])
        np.testing.assert_array_equal(deq[:, 0], 1.0)


def test_dyn_error_bound_zero_block_and_scale():
    rng = np.random.default_rng(6)
    m = rng.standard_normal((4, 256)) * 1e-3
    m[1, 64:128] = 0.0
    q, s = q8.quant_dyn_signed(m)
    assert q.dtype == np.uint8 and s.shape == (4, 4)
    np.testing.assert_array_equal(s, np.max(np.abs(m.astype(np.float32)), axis=-1).reshape(4, 4)
                                  if False else np.abs(m.astype(np.float32)).reshape(4, 4, 64).max(-1))
    assert s[1, 1] == 0 and np.all(q[1, 64:128] == 0)
    deq = q8.dequant_dyn_signed(q, s)
    # error <= half the gap to the neighbouring code, in units of the block scale
    t = q8.DYN_SIGNED.astype(np.float64)
    gap = np.maximum(np.diff(t, prepend=0.0), np.diff(t, append=1.0))
    k = (q & 0x7F).astype(np.int64)
    bound = 0.5 * gap[k] * np.repeat(s.astype(np.float64), 64, axis=1) * (1 + 1e-6) + 1e-30
    assert np.all(np.abs(deq - m) <= bound + np.abs(m) * 2 ** -23)
    v = m ** 2
    qv, sv = q8.quant_dyn_unsigned(v)
    assert np.all(q8.dequant_dyn_unsigned(qv, sv) >= 0)


def test_dyn_keeps_small_values_a_linear_code_loses():
    """The reason for a dynamic code: next to a block outlier 1000x larger, small
    moments keep their size (8 codes per decade there: relative error ~10%) where
    127 linear levels round them to 0."""
    rng = np.random.default_rng(7)
    m = rng.standard_normal((16, 64)) * 1e-4
    m[:, 0] = 1e-1
    ql, sl = q8.quant_signed(m)
    qd, sd = q8.quant_dyn_signed(m)
    lin = q8.dequant_signed(ql, sl)[:, 1:]
    dyn = q8.dequant_dyn_signed(qd, sd)[:, 1:]
    assert np.mean(lin == 0) > 0.9
    rel = np.abs(dyn - m[:, 1:]) / np.abs(m[:, 1:])
    assert np.all(dyn != 0) and np.median(rel) < 0.15 and np.max(rel) < 0.6


def test_dyn_rank_orders_codes_by_value():
    b = np.arange(256, dtype=np.uint8)
    r = q8.dyn_rank(b, signed=True)
    val = np.where(b & 0x80, -1.0, 1.0) * q8.DYN_SIGNED[b & 0x7F]
    ok = b != 0x80
    order = np.argsort(val[ok], kind="stable")
    assert np.all(np.diff(r[ok][order]) >= 0)
