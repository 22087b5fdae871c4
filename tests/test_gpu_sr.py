"""Statistics of the GPU path's stochastic rounding (the pages: the bfloat16 weight
write-back uses stochastic rounding so that updates below one ulp accumulate
without bias and the bfloat16 "dead zone" is avoided; §2 "Precision and fidelity").

Every weight of a 128x128 layer starts at 1.0 and takes SGD steps (lr 1, no decay)
with a gradient of exactly c = 1.203125 * 2^-10 (X = 1, dY = c, one token), a
third of the bfloat16 ulp 2^-8 just below 1.0. Each element rounds with its own
counter-hash bits, so the 16384 elements are 16384 rounding trials per step.
"""
import numpy as np
import pytest
import torch

from synth import bf16_bits_from_f32
from tests import _parity as P

pytestmark = pytest.mark.gpu

N_OUT = N_IN = 128
ULP = 2.0 ** -8                     # bfloat16 spacing in [0.5, 1)
C = 1.203125 * 2.0 ** -10           # the gradient: exact in bfloat16, 0.3008 ulp


def _run(steps, sr, seed):
    import optimizer_gemm_amd as f
    print(f"[case] SR statistics: steps={steps} sr={sr} seed={seed}", flush=True)
    W = P.dev_bf16(bf16_bits_from_f32(np.ones((N_OUT, N_IN), np.float32)))
    X = P.dev_bf16(bf16_bits_from_f32(np.ones((1, N_IN), np.float32)))
    dY = P.dev_bf16(bf16_bits_from_f32(np.full((1, N_OUT), C, np.float32)))
    hyper = dict(lr=1.0, weight_decay=0.0, stochastic_round=int(sr))
    for t in range(1, steps + 1):
        f.wgrad_step(X, dY, W, None, None, "sgd", hyper, t, seed)
    torch.cuda.synchronize()
    return W.float().cpu().numpy().astype(np.float64)


def test_sr_unbiased_over_16384_trials():
    # one step: each weight becomes 1.0 or 1 - ulp, and the mean is 1 - c within 4 standard errors
    w = _run(1, True, 0x5EED_5151)
    assert set(np.unique(w)) <= {1.0, 1.0 - ULP}
    p = C / ULP
    se = ULP * np.sqrt(p * (1 - p) / w.size)
    assert abs(w.mean() - (1.0 - C)) <= 4 * se, (w.mean(), 1.0 - C, se)


def test_dead_zone_rne_stalls_sr_drifts():
    # 20 steps of a third of an ulp: round-to-nearest never moves the weights; stochastic
    # rounding moves them down by 20 c on average (each step a Bernoulli(c / ulp) drop)
    w_rne = _run(20, False, 0x5EED_5152)
    assert np.all(w_rne == 1.0)
    w_sr = _run(20, True, 0x5EED_5153)
    p = C / ULP
    se = ULP * np.sqrt(20 * p * (1 - p) / w_sr.size)
    assert abs(w_sr.mean() - (1.0 - 20 * C)) <= 4 * se, (w_sr.mean(), 1.0 - 20 * C, se)
    drops = np.rint((1.0 - w_sr) / ULP)
    assert np.all(drops == (1.0 - w_sr) / ULP) and drops.min() >= 0 and drops.max() <= 20
