"""Pins for the oracle's counter-based RNG and stochastic rounding (no GPU).

The pages require unbiased stochastic rounding of the bfloat16 weight
write-back (§2 "Precision and fidelity") without giving a rule; the oracle's
reading is SplitMix64 on (seed, step, element index) and the bit-add rounding.
Pins: the published SplitMix64 sequence, the counting identity that makes the
rounding unbiased, a value-based statement of stochastic rounding, and the
special values.
"""
import os

import numpy as np
import pytest

from oracle import rounding

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _published():
    vals, seed = [], None
    for line in open(os.path.join(GOLDEN, "splitmix64_published.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("seed"):
            seed = int(line.split()[1])
        else:
            vals.append(int(line))
    return seed, vals


def test_splitmix64_published_sequence_both_forms():
    seed, vals = _published()
    assert rounding.splitmix64_py(seed, len(vals)) == vals
    got = rounding.splitmix64_at(seed, np.arange(len(vals), dtype=np.uint64))
    assert [int(x) for x in got] == vals


def test_counter_jump_equals_sequential_stepping():
    rng = np.random.default_rng(0)
    for seed in (0, 0x5EED0001, (1 << 64) - 1):
        cs = rng.integers(0, 4000, size=20)
        seq = rounding.splitmix64_py(seed, int(cs.max()) + 1)
        got = rounding.splitmix64_at(seed, cs.astype(np.uint64))
        assert [int(x) for x in got] == [seq[c] for c in cs]


def test_counter_layout():
    c = rounding.counters(3, np.array([0, 5, (1 << 32) - 1], dtype=np.uint64))
    assert [int(x) for x in c] == [3 << 32, (3 << 32) | 5, (3 << 32) | ((1 << 32) - 1)]
    with pytest.raises(ValueError):
        rounding.counters(1, np.array([1 << 32], dtype=np.uint64))


def test_element_index_row_major():
    idx = rounding.element_index(np.array([0, 2]), 5)
    np.testing.assert_array_equal(idx, [[0, 1, 2, 3, 4], [10, 11, 12, 13, 14]])


def test_rand16_frozen_known_answers():
    for line in open(os.path.join(GOLDEN, "rand16_kat.txt")):
        if line.startswith("#"):
            continue
        seed, step, idx, r = (int(x) for x in line.split())
        assert int(rounding.rand16(seed, step, np.array([idx], dtype=np.uint64))[0]) == r


def test_rand16_uniform_buckets():
    r = rounding.rand16(0x5EED0001, 7, np.arange(1 << 20, dtype=np.uint64))
    counts = np.bincount(r >> 12, minlength=16)
    expect = (1 << 20) / 16
    chi2 = float(np.sum((counts - expect) ** 2 / expect))
    assert chi2 < 45.0  # 15 dof; p ~ 1e-4
    assert r.max() < 65536


def test_sr_counting_identity():
    # For every x, exactly low16(bits(x)) of the 65536 values of r16 round the magnitude up.
    r16 = np.arange(65536, dtype=np.uint32)
    for bits in (0x3F800000, 0x3F800001, 0x3F80FFFF, 0xBF812345, 0x00012345, 0x7F7F8000, 0x4049C000):
        x = np.full(65536, np.uint32(bits)).view(np.float32)
        out = rounding.sr_bf16(x, r16).astype(np.uint32)
        up = int(np.sum(out != (bits >> 16)))
        assert up == (bits & 0xFFFF)
        assert np.all((out == (bits >> 16)) | (out == (bits >> 16) + 1))


def test_sr_matches_value_based_definition():
    # Round |x| up to the next bfloat16 with probability (|x|-|lo|)/(|hi|-|lo|), where lo is x
    # truncated toward zero; with r16 uniform on [0, 65536) "up" means r16 >= 65536*(1-p).
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    r16 = rng.integers(0, 65536, size=x.size).astype(np.uint32)
    got = rounding.bf16_to_f64(rounding.sr_bf16(x, r16))
    ax = np.abs(x.astype(np.float64))
    lo = rounding.bf16_to_f64((np.abs(x).view(np.uint32) >> 16).astype(np.uint16))
    hi = rounding.bf16_to_f64(((np.abs(x).view(np.uint32) >> 16) + 1).astype(np.uint16))
    p = (ax - lo) / (hi - lo)
    up = r16.astype(np.float64) >= 65536.0 * (1.0 - p)
    expect = np.sign(x) * np.where(up & (p > 0), hi, lo)
    np.testing.assert_array_equal(got, expect)


def test_sr_zero_r_truncates_toward_zero():
    x = np.array([1.9999, -1.9999, 3.0e-5, -7.77e7], dtype=np.float32)
    out = rounding.sr_bf16(x, np.zeros(4, dtype=np.uint32))
    np.testing.assert_array_equal(out, (x.view(np.uint32) >> 16).astype(np.uint16))


def test_sr_special_values():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, -0.0, 0.0, np.finfo(np.float32).max], dtype=np.float32)
    x[1] = np.float32(-np.nan)
    x_bits = x.view(np.uint32).copy()
    x_bits[1] = 0xFFFFFFFF  # a negative NaN whose mantissa would wrap without the NaN rule
    x = x_bits.view(np.float32)
    out = rounding.sr_bf16(x, np.full(7, 0xFFFF, dtype=np.uint32))
    assert out[0] == 0x7FC0 and out[1] == 0xFFC0
    assert out[2] == 0x7F80 and out[3] == 0xFF80
    assert out[4] == 0x8000 and out[5] == 0x0000
    assert out[6] == 0x7F80  # FLT_MAX may round up to +Inf: valid stochastic rounding


def test_sr_frozen_known_answers():
    for line in open(os.path.join(GOLDEN, "sr_bf16_kat.txt")):
        if line.startswith("#"):
            continue
        xb, r, b = (int(v, 16) for v in line.split())
        x = np.array([xb], dtype=np.uint32).view(np.float32)
        assert int(rounding.sr_bf16(x, np.array([r]))[0]) == b


def test_sr_exactly_unbiased_over_all_r16():
    r16 = np.arange(65536, dtype=np.uint32)
    for xv in (1.003, -0.0200023, 1e-3 + 3e-9, 123.456):
        x = np.full(65536, np.float32(xv))
        mean = np.mean(rounding.bf16_to_f64(rounding.sr_bf16(x, r16)))
        assert mean == float(np.float32(xv))


def test_sr_unbiased_monte_carlo_1e4_trials():
    x = np.float32(1.003)
    n = 10_000
    r16 = rounding.rand16(0x5EED0002, 1, np.arange(n, dtype=np.uint64))
    vals = rounding.bf16_to_f64(rounding.sr_bf16(np.full(n, x), r16))
    lo = rounding.bf16_to_f64(np.array([x.view(np.uint32) >> 16], dtype=np.uint16))[0]
    ulp = 2.0 ** -7
    p = (float(x) - lo) / ulp
    assert abs(vals.mean() - float(x)) <= 4 * ulp * np.sqrt(p * (1 - p) / n)


def test_dead_zone_rne_stalls_sr_drifts():
    # Add a quarter-ulp update 400 times to 1.0 in bfloat16.
    steps, delta = 400, 0.25 * 2.0 ** -7
    w_rne = np.float64(1.0)
    w_sr = np.float64(1.0)
    for k in range(steps):
        x = np.array([w_rne + delta], dtype=np.float32)
        u = x.view(np.uint32)
        w_rne = rounding.bf16_to_f64(((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16))[0]
        xs = np.array([w_sr + delta], dtype=np.float32)
        w_sr = rounding.bf16_to_f64(rounding.sr_bf16(xs, rounding.rand16(9, k + 1, np.array([0]))))[0]
    assert w_rne == 1.0
    expect = 1.0 + steps * delta  # 1.78125
    # standard deviation of the sum of 400 rounding errors is at most 0.5 ulp * sqrt(400) ~ 0.04
    assert abs(w_sr - expect) < 0.2
