"""Pins for the oracle's OCP FP8 decoding (no GPU).

The OCP 8-bit floating point specification fixes both formats; the pins are the
values that specification tabulates (largest finite, smallest normal and
subnormal, the special encodings) and a second, independent implementation:
PyTorch's float8_e4m3fn / float8_e5m2 conversions, compared on all 256 codes.
"""
import numpy as np
import pytest
import torch

from oracle import fp8, gemm


def _torch_decode(fmt):
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dt).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", fp8.FORMATS)
def test_all_codes_match_torch(fmt):
    ours = fp8.decode(np.arange(256, dtype=np.uint8), fmt)
    ref = _torch_decode(fmt)
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[~both_nan], ref[~both_nan])


def test_e4m3_tabulated_values():
    d = lambda c: float(fp8.decode(np.array([c], dtype=np.uint8), "e4m3")[0])
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals
    assert d(0x38) == 1.0 and d(0x00) == 0.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))           # no infinities, one NaN pattern
    assert sum(np.isnan(fp8.decode(np.arange(256, dtype=np.uint8), "e4m3"))) == 2


def test_e5m2_tabulated_values():
    d = lambda c: float(fp8.decode(np.array([c], dtype=np.uint8), "e5m2")[0])
    assert d(0x7B) == 57344.0                              # largest finite
    assert d(0x7C) == np.inf and d(0xFC) == -np.inf
    assert all(np.isnan(d(c)) for c in (0x7D, 0x7E, 0x7F))
    assert d(0x04) == 2.0 ** -14 and d(0x01) == 2.0 ** -16
    assert d(0x3C) == 1.0


def test_dequantised_gradient_is_scaled_product():
    # dW from codes and scales equals the gradient of the decoded values times sx*sdy
    rng = np.random.default_rng(3)
    X = rng.integers(0, 0x7F, size=(40, 24), dtype=np.uint8)     # finite positive and zero e4m3 codes
    dY = rng.integers(0, 0x7B, size=(40, 16), dtype=np.uint8)    # finite e5m2 codes
    sx, sdy = 0.125, 3.0
    g = gemm.wgrad(fp8.dequant(X, "e4m3", sx), fp8.dequant(dY, "e5m2", sdy))
    g0 = gemm.wgrad(fp8.decode(X, "e4m3"), fp8.decode(dY, "e5m2"))
    np.testing.assert_allclose(g, g0 * sx * sdy, rtol=1e-15)
