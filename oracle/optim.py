"""The eight element-wise optimizers, in float64 (oracle).

The pages name the set (§3 "Contributions", generality paragraph: AdamW, NAdam,
RAdam, Lion, RMSprop, AdaGrad, SGD, SGD-momentum) and state that each update of
a weight depends only on that weight's coordinate (§2 "Precision and fidelity",
exactness paragraph), but print no equations. The baseline the pages compare
against is a fused AdamW (§4 "Experimental results"). Reading used here: the
textbook algorithms in the conventions of PyTorch's torch.optim (decoupled,
lr-scaled weight decay for AdamW and Lion; coupled L2 decay g += wd*theta for
the other six), with bias corrections on the 1-based step t.

Every function works element-wise on float64 arrays, so it applies equally to a
whole weight, a 128x128 tile or a sampled row.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

OPTIMIZERS = ("adamw", "sgd", "sgd_momentum", "lion", "rmsprop", "adagrad", "nadam", "radam")

# Which moment slots an optimizer keeps: "m" is the first slot, "v" the second.
SLOTS: Dict[str, Tuple[str, ...]] = {
    "adamw": ("m", "v"), "sgd": (), "sgd_momentum": ("m",), "lion": ("m",),
    "rmsprop": ("v",), "adagrad": ("v",), "nadam": ("m", "v"), "radam": ("m", "v"),
}

_BASE = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, momentum=0.0,
             dampening=0.0, nesterov=False, alpha=0.99, lr_decay=0.0, momentum_decay=4e-3)

# Default hyper-parameters of the optimizer sweep (AdamW values are the workload's).
DEFAULTS: Dict[str, Dict[str, float]] = {
    "adamw": dict(_BASE, weight_decay=0.01),
    "sgd": dict(_BASE),
    "sgd_momentum": dict(_BASE, momentum=0.9),
    "lion": dict(_BASE, lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.1),
    "rmsprop": dict(_BASE, alpha=0.99, eps=1e-8),
    "adagrad": dict(_BASE, eps=1e-10),
    "nadam": dict(_BASE),
    "radam": dict(_BASE),
}


def hyper(opt: str, **over) -> Dict[str, float]:
    if opt not in DEFAULTS:
        raise ValueError(f"unknown optimizer {opt!r}")
    h = dict(DEFAULTS[opt])
    for k, val in over.items():
        if k not in h:
            raise KeyError(k)
        h[k] = val
    return h


def nadam_mu(beta1: float, psi: float, k: int) -> float:
    """NAdam momentum schedule mu_k = beta1 * (1 - 0.5 * 0.96**(k * psi))."""
    return beta1 * (1.0 - 0.5 * 0.96 ** (k * psi))


def radam_rho(beta2: float, t: int) -> Tuple[float, float]:
    """RAdam (rho_inf, rho_t): length of the approximated simple moving average."""
    rho_inf = 2.0 / (1.0 - beta2) - 1.0
    bc2 = 1.0 - beta2 ** t
    return rho_inf, rho_inf - 2.0 * t * beta2 ** t / bc2


def update(opt: str, theta: np.ndarray, g: np.ndarray, m: Optional[np.ndarray], v: Optional[np.ndarray],
           hp: Dict[str, float], t: int):
    """One optimizer step on float64 arrays; returns (theta, m, v) (unused slots None).

    theta: weights, g: gradient (already complete for these coordinates),
    m / v: the optimizer's moment slots as listed in SLOTS, t: 1-based step.
    """
    if t < 1:
        raise ValueError("step is 1-based")
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = None if m is None else np.asarray(m, dtype=np.float64)
    v = None if v is None else np.asarray(v, dtype=np.float64)
    lr, b1, b2, eps, wd = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]

    if opt == "adamw":
        # Loshchilov & Hutter: decoupled decay scaled by lr, then Adam with bias correction.
        theta = theta * (1.0 - lr * wd)
        m = b1 * m + (1.0 - b1) * g
        v = b2 * v + (1.0 - b2) * g * g
        mhat = m / (1.0 - b1 ** t)
        vhat = v / (1.0 - b2 ** t)
        theta = theta - lr * mhat / (np.sqrt(vhat) + eps)
        return theta, m, v

    if opt == "sgd":
        d = g + wd * theta
        return theta - lr * d, None, None

    if opt == "sgd_momentum":
        mu, damp = hp["momentum"], hp["dampening"]
        d = g + wd * theta
        # The momentum buffer starts as the first gradient itself (no dampening on step 1).
        b = d.copy() if t == 1 else mu * m + (1.0 - damp) * d
        step_dir = d + mu * b if hp["nesterov"] else b
        return theta - lr * step_dir, b, None

    if opt == "lion":
        # Chen et al. 2023: sign of the beta1 interpolation; the state tracks with beta2.
        c = b1 * m + (1.0 - b1) * g
        theta = theta * (1.0 - lr * wd) - lr * np.sign(c)
        m = b2 * m + (1.0 - b2) * g
        return theta, m, None

    if opt == "rmsprop":
        a = hp["alpha"]
        d = g + wd * theta
        v = a * v + (1.0 - a) * d * d
        return theta - lr * d / (np.sqrt(v) + eps), None, v

    if opt == "adagrad":
        d = g + wd * theta
        lr_t = lr / (1.0 + (t - 1) * hp["lr_decay"])
        v = v + d * d
        return theta - lr_t * d / (np.sqrt(v) + eps), None, v

    if opt == "nadam":
        psi = hp["momentum_decay"]
        d = g + wd * theta
        mu_t = nadam_mu(b1, psi, t)
        mu_n = nadam_mu(b1, psi, t + 1)
        prod_t = math.prod(nadam_mu(b1, psi, k) for k in range(1, t + 1))
        prod_n = prod_t * mu_n
        m = b1 * m + (1.0 - b1) * d
        v = b2 * v + (1.0 - b2) * d * d
        denom = np.sqrt(v / (1.0 - b2 ** t)) + eps
        theta = theta - lr * (1.0 - mu_t) / (1.0 - prod_t) * d / denom \
                      - lr * mu_n / (1.0 - prod_n) * m / denom
        return theta, m, v

    if opt == "radam":
        d = g + wd * theta
        m = b1 * m + (1.0 - b1) * d
        v = b2 * v + (1.0 - b2) * d * d
        bc1 = 1.0 - b1 ** t
        bc2 = 1.0 - b2 ** t
        rho_inf, rho_t = radam_rho(b2, t)
        mhat = m / bc1
        if rho_t > 5.0:
            r = math.sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t))
            theta = theta - lr * r * mhat * math.sqrt(bc2) / (np.sqrt(v) + eps)
        else:
            theta = theta - lr * mhat
        return theta, m, v

    raise ValueError(f"unknown optimizer {opt!r}")
