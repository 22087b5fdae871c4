"""Pins for the oracle's eight optimizers (no GPU).

The pages list the optimizer set (§3 Contributions, generality) without
equations; the oracle follows the textbook algorithms as torch.optim implements
them. Two kinds of pins:
  * torch.optim's own float64 implementation, run on the same gradients, for
    the seven optimizers torch provides (Lion has none here);
  * closed forms that follow from the algorithms' definitions.
"""
import math

import numpy as np
import pytest
import torch

from oracle import optim

STEPS = 12  # RAdam switches to the rectified branch at t = 6 with beta2 = 0.999


def _torch_opt(name, p, hp):
    if name == "adamw":
        return torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                 weight_decay=hp["weight_decay"], foreach=False)
    if name in ("sgd", "sgd_momentum"):
        return torch.optim.SGD([p], lr=hp["lr"], momentum=hp["momentum"], dampening=hp["dampening"],
                               nesterov=hp["nesterov"], weight_decay=hp["weight_decay"], foreach=False)
    if name == "rmsprop":
        return torch.optim.RMSprop([p], lr=hp["lr"], alpha=hp["alpha"], eps=hp["eps"],
                                   weight_decay=hp["weight_decay"], foreach=False)
    if name == "adagrad":
        return torch.optim.Adagrad([p], lr=hp["lr"], lr_decay=hp["lr_decay"], eps=hp["eps"],
                                   weight_decay=hp["weight_decay"], foreach=False)
    if name == "nadam":
        return torch.optim.NAdam([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                 weight_decay=hp["weight_decay"], momentum_decay=hp["momentum_decay"],
                                 foreach=False)
    if name == "radam":
        return torch.optim.RAdam([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                 weight_decay=hp["weight_decay"], foreach=False)
    raise ValueError(name)


CASES = [
    ("adamw", {}),
    ("adamw", dict(weight_decay=0.1, lr=3e-3, beta1=0.8, beta2=0.95)),
    ("sgd", {}),
    ("sgd", dict(weight_decay=0.05)),
    ("sgd_momentum", {}),
    ("sgd_momentum", dict(weight_decay=0.01, dampening=0.3)),
    ("sgd_momentum", dict(nesterov=True, weight_decay=0.02)),
    ("rmsprop", {}),
    ("rmsprop", dict(weight_decay=0.02, alpha=0.9)),
    ("adagrad", {}),
    ("adagrad", dict(weight_decay=0.01, lr_decay=0.05)),
    ("nadam", {}),
    ("nadam", dict(weight_decay=0.01, momentum_decay=0.01)),
    ("radam", {}),
    ("radam", dict(weight_decay=0.01)),
]


@pytest.mark.parametrize("name,over", CASES)
def test_matches_torch_optim_float64(name, over):
    hp = optim.hyper(name, **over)
    rng = np.random.default_rng(11)
    theta0 = rng.standard_normal(257) * 0.02
    grads = [rng.standard_normal(257) * 1e-2 * (1 + 0.5 * k) for k in range(STEPS)]
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)  # keep torch's per-step scalars in float64 too
    try:
        p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
        opt = _torch_opt(name, p, hp)
        theta = theta0.copy()
        slots = optim.SLOTS[name]
        m = np.zeros_like(theta) if "m" in slots else None
        v = np.zeros_like(theta) if "v" in slots else None
        for t in range(1, STEPS + 1):
            g = grads[t - 1]
            p.grad = torch.tensor(g, dtype=torch.float64)
            opt.step()
            theta, m, v = optim.update(name, theta, g, m, v, hp, t)
            np.testing.assert_allclose(theta, p.detach().numpy(), rtol=1e-12, atol=1e-15,
                                       err_msg=f"{name} step {t}")
    finally:
        torch.set_default_dtype(old)


def test_adamw_first_step_closed_form():
    hp = optim.hyper("adamw")
    g = np.array([3e-3, -2e-5, 0.0, 1e-9])
    th = np.array([0.01, -0.02, 0.03, 0.0])
    out, m, v = optim.update("adamw", th, g, np.zeros(4), np.zeros(4), hp, 1)
    lr, lam, eps = hp["lr"], hp["weight_decay"], hp["eps"]
    expect = th * (1 - lr * lam) - lr * g / (np.abs(g) + eps)
    np.testing.assert_allclose(out, expect, rtol=1e-12)
    np.testing.assert_allclose(m, (1 - hp["beta1"]) * g)
    np.testing.assert_allclose(v, (1 - hp["beta2"]) * g * g)


def test_adamw_constant_gradient_closed_form():
    hp = optim.hyper("adamw", weight_decay=0.0)
    g = np.array([1e-3, -4e-2, 7.0])
    th0 = np.array([0.5, -0.25, 0.0])
    th, m, v = th0, np.zeros(3), np.zeros(3)
    for t in range(1, 9):
        th, m, v = optim.update("adamw", th, g, m, v, hp, t)
    # bias correction makes mhat = g and vhat = g^2 exactly for a constant gradient
    np.testing.assert_allclose(th, th0 - 8 * hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-12)


def test_sgd_closed_form():
    hp = optim.hyper("sgd")
    g = np.array([1.0, -2.0])
    th, m, v = optim.update("sgd", np.array([0.1, 0.2]), g, None, None, hp, 3)
    np.testing.assert_allclose(th, np.array([0.1, 0.2]) - 1e-3 * g)
    assert m is None and v is None


def test_sgd_momentum_constant_gradient_closed_form():
    hp = optim.hyper("sgd_momentum")
    mu, lr = hp["momentum"], hp["lr"]
    g = np.array([2.0, -1.0])
    th0 = np.array([1.0, 1.0])
    th, b = th0, np.zeros(2)
    for t in range(1, 7):
        th, b, _ = optim.update("sgd_momentum", th, g, b, None, hp, t)
        np.testing.assert_allclose(b, g * (1 - mu ** t) / (1 - mu), rtol=1e-13)
    total = sum((1 - mu ** k) / (1 - mu) for k in range(1, 7))
    np.testing.assert_allclose(th, th0 - lr * g * total, rtol=1e-13)


def test_lion_first_step_and_constant_gradient():
    hp = optim.hyper("lion")
    lr, lam = hp["lr"], hp["weight_decay"]
    g = np.array([0.3, -1e-7, 0.0])
    th0 = np.array([0.2, -0.1, 0.05])
    th, m, _ = optim.update("lion", th0, g, np.zeros(3), None, hp, 1)
    np.testing.assert_allclose(th, th0 * (1 - lr * lam) - lr * np.sign(g), rtol=1e-14)
    # sign(0) = 0: a zero gradient only decays
    assert th[2] == pytest.approx(th0[2] * (1 - lr * lam), rel=1e-15)
    th, m = th0, np.zeros(3)
    for t in range(1, 6):
        th, m, _ = optim.update("lion", th, g, m, None, hp, t)
    decay = 1 - lr * lam
    expect = th0 * decay ** 5 - lr * np.sign(g) * sum(decay ** k for k in range(5))
    np.testing.assert_allclose(th, expect, rtol=1e-13)


def test_lion_interpolation_uses_beta1_and_state_uses_beta2():
    # g1 = 1 then g2 = -0.5: m1 = (1-b2)*1 = 0.01; c2 = b1*m1 + (1-b1)*g2 = -0.041 < 0.
    # A swapped beta (c with b2, or m with b1) would give c2 > 0.
    hp = optim.hyper("lion", weight_decay=0.0)
    th, m, _ = optim.update("lion", np.zeros(1), np.array([1.0]), np.zeros(1), None, hp, 1)
    np.testing.assert_allclose(m, [0.01])
    th, m, _ = optim.update("lion", th, np.array([-0.5]), m, None, hp, 2)
    np.testing.assert_allclose(th, [-hp["lr"] + hp["lr"]], atol=1e-18)
    np.testing.assert_allclose(m, [0.99 * 0.01 + 0.01 * -0.5])


def test_rmsprop_first_step_closed_form():
    hp = optim.hyper("rmsprop")
    g = np.array([2e-3, -5e-4])
    th, _, v = optim.update("rmsprop", np.zeros(2), g, None, np.zeros(2), hp, 1)
    np.testing.assert_allclose(th, -hp["lr"] * g / (math.sqrt(1 - hp["alpha"]) * np.abs(g) + hp["eps"]))
    # about ten lr-sized steps for alpha = 0.99
    assert np.all(np.abs(np.abs(th) / hp["lr"] - 10.0) < 5e-3)


def test_adagrad_constant_gradient_closed_form():
    hp = optim.hyper("adagrad")
    g = np.array([0.5, -3.0])
    th, s = np.zeros(2), np.zeros(2)
    for t in range(1, 5):
        th, _, s = optim.update("adagrad", th, g, None, s, hp, t)
    expect = -sum(hp["lr"] * g / (math.sqrt(k) * np.abs(g) + hp["eps"]) for k in range(1, 5))
    np.testing.assert_allclose(th, expect, rtol=1e-13)


def test_nadam_first_step_coefficient():
    hp = optim.hyper("nadam")
    g = np.array([1e-2, -3e-3])
    th, _, _ = optim.update("nadam", np.zeros(2), g, np.zeros(2), np.zeros(2), hp, 1)
    mu1 = 0.9 * (1 - 0.5 * 0.96 ** 0.004)
    mu2 = 0.9 * (1 - 0.5 * 0.96 ** 0.008)
    coef = 1 + mu2 * (1 - 0.9) / (1 - mu1 * mu2)
    assert mu1 == pytest.approx(0.450073, abs=1e-6) and mu2 == pytest.approx(0.450147, abs=1e-6)
    assert coef == pytest.approx(1.056452, abs=1e-6)
    np.testing.assert_allclose(th, -coef * hp["lr"] * g / (np.abs(g) + hp["eps"]), rtol=1e-9)


def test_radam_rho_values_and_unrectified_steps():
    hp = optim.hyper("radam")
    rhos = [optim.radam_rho(0.999, t)[1] for t in range(1, 7)]
    np.testing.assert_allclose(rhos, [1.0, 1.9995, 2.9987, 3.9975, 4.9960, 5.9942], atol=1e-4)
    g = np.array([0.1, -0.2])
    th, m, v = np.zeros(2), np.zeros(2), np.zeros(2)
    th, m, v = optim.update("radam", th, g, m, v, hp, 1)
    np.testing.assert_allclose(th, -hp["lr"] * g, rtol=1e-14)  # step 1 is plain SGD with m/bc1 = g
    for t in range(2, 6):
        prev = th
        th, m, v = optim.update("radam", th, g, m, v, hp, t)
        np.testing.assert_allclose(th, prev - hp["lr"] * m / (1 - 0.9 ** t), rtol=1e-14)


def test_bad_arguments():
    with pytest.raises(ValueError):
        optim.update("adamw", np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), optim.hyper("adamw"), 0)
    with pytest.raises(ValueError):
        optim.hyper("adam")
