"""The eight element-wise optimizers, float64 (oracle; test infrastructure only).

FORGE explainer (gist.science), Technical Summary section 3 "Key
Contributions" names eight fully fused element-wise optimizers: AdamW, NAdam,
RAdam, Lion, RMSprop, AdaGrad, SGD and SGD-momentum; section 2 "Precision and
Fidelity" states that for element-wise-separable rules the tile update equals
the full-gradient step.  The pages give no formulas, so each rule is its
published form, with the common library defaults where the publication
leaves a choice:

  AdamW   Loshchilov & Hutter, "Decoupled Weight Decay Regularization".
  NAdam   Dozat, "Incorporating Nesterov Momentum into Adam", with the
          momentum schedule mu_t = beta1 * (1 - 0.5 * 0.96^(t * psi)).
  RAdam   Liu et al., "On the Variance of the Adaptive Learning Rate and
          Beyond"; rectified branch when rho_t > 5, eps added to sqrt(v).
  Lion    Chen et al., "Symbolic Discovery of Optimization Algorithms".
  RMSprop Hinton's lecture form, non-centred, no momentum.
  AdaGrad Duchi et al., accumulator starting at 0, no learning-rate decay.
  SGD, SGD with heavy-ball momentum (dampening 0, not Nesterov).

Weight decay: AdamW and Lion decay the weight directly ("decoupled", applied
to the weight before this step's update); the others add wd * W to the
gradient ("coupled L2").  hyper.wd_mode = 1 forces decoupled, 2 forces L2.

Hyper-parameters arrive as fp32 (that is what the library's interface
carries); the oracle promotes those exact fp32 values to float64.  Per-step
scalars (bias corrections, rho_t, r_t, the NAdam momentum products) are
float64 functions of the step count t >= 1.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

NAMES = ("adamw", "nadam", "radam", "lion", "rmsprop", "adagrad", "sgd", "sgd_momentum")

# which moment buffers each rule keeps: m is signed, v is non-negative
STATES = {
    "adamw": ("m", "v"), "nadam": ("m", "v"), "radam": ("m", "v"),
    "lion": ("m",), "rmsprop": ("v",), "adagrad": ("v",),
    "sgd": (), "sgd_momentum": ("m",),
}


def f32(x) -> float:
    return float(np.float32(x))


def hyper64(h) -> Dict[str, float]:
    return dict(lr=f32(h.lr), beta1=f32(h.beta1), beta2=f32(h.beta2), eps=f32(h.eps),
                wd=f32(h.weight_decay), wd_mode=int(h.wd_mode), momentum=f32(h.momentum),
                alpha=f32(h.alpha), psi=f32(h.momentum_decay))


def decoupled(opt: str, wd_mode: int) -> bool:
    if wd_mode == 1:
        return True
    if wd_mode == 2:
        return False
    return opt in ("adamw", "lion")


def nadam_mu(beta1: float, psi: float, t: int) -> float:
    return beta1 * (1.0 - 0.5 * 0.96 ** (t * psi))


def step_scalars(opt: str, h, t: int) -> Dict[str, float]:
    """Per-step scalars of rule `opt` at step t >= 1, in float64."""
    if t < 1:
        raise ValueError("step count starts at 1")
    p = hyper64(h)
    b1, b2 = p["beta1"], p["beta2"]
    s: Dict[str, float] = {}
    if opt in ("adamw", "nadam", "radam"):
        s["bc1"] = 1.0 - b1 ** t
        s["bc2"] = 1.0 - b2 ** t
    if opt == "nadam":
        prod = 1.0
        for i in range(1, t + 1):
            prod *= nadam_mu(b1, p["psi"], i)
        s["mu"] = nadam_mu(b1, p["psi"], t)
        s["mu_next"] = nadam_mu(b1, p["psi"], t + 1)
        s["prod"] = prod
        s["prod_next"] = prod * s["mu_next"]
    if opt == "radam":
        rho_inf = 2.0 / (1.0 - b2) - 1.0
        rho_t = rho_inf - 2.0 * t * b2 ** t / (1.0 - b2 ** t)
        s["rho_inf"], s["rho_t"] = rho_inf, rho_t
        s["rectified"] = rho_t > 5.0
        if s["rectified"]:
            s["r"] = math.sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf
                               / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t))
    return s


def update(opt: str, h, t: int, g: np.ndarray, W: np.ndarray,
           m: Optional[np.ndarray] = None, v: Optional[np.ndarray] = None
           ) -> Tuple[np.ndarray, Optional[np.ndarray], Optional[np.ndarray]]:
    """One step of rule `opt` on float64 arrays; returns (W_new, m_new, v_new).

    g is the full gradient of each element, W the weight before the step,
    m and v the moments before the step (zeros at t = 1).
    """
    p = hyper64(h)
    s = step_scalars(opt, h, t)
    lr, b1, b2, eps, wd = p["lr"], p["beta1"], p["beta2"], p["eps"], p["wd"]
    g = np.asarray(g, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    dec = decoupled(opt, p["wd_mode"])
    if not dec and wd != 0.0:
        g = g + wd * W
    Wd = W * (1.0 - lr * wd) if (dec and wd != 0.0) else W
    m_new = v_new = None

    if opt == "adamw":
        m_new = b1 * m + (1.0 - b1) * g
        v_new = b2 * v + (1.0 - b2) * g * g
        denom = np.sqrt(v_new / s["bc2"]) + eps
        W_new = Wd - lr * (m_new / s["bc1"]) / denom
    elif opt == "nadam":
        m_new = b1 * m + (1.0 - b1) * g
        v_new = b2 * v + (1.0 - b2) * g * g
        denom = np.sqrt(v_new / s["bc2"]) + eps
        c_g = lr * (1.0 - s["mu"]) / (1.0 - s["prod"])
        c_m = lr * s["mu_next"] / (1.0 - s["prod_next"])
        W_new = Wd - c_g * g / denom - c_m * m_new / denom
    elif opt == "radam":
        m_new = b1 * m + (1.0 - b1) * g
        v_new = b2 * v + (1.0 - b2) * g * g
        mhat = m_new / s["bc1"]
        if s["rectified"]:
            adapt = math.sqrt(s["bc2"]) / (np.sqrt(v_new) + eps)
            W_new = Wd - lr * s["r"] * mhat * adapt
        else:
            W_new = Wd - lr * mhat
    elif opt == "lion":
        c = b1 * m + (1.0 - b1) * g
        W_new = Wd - lr * np.sign(c)
        m_new = b2 * m + (1.0 - b2) * g
    elif opt == "rmsprop":
        a = p["alpha"]
        v_new = a * v + (1.0 - a) * g * g
        W_new = Wd - lr * g / (np.sqrt(v_new) + eps)
    elif opt == "adagrad":
        v_new = v + g * g
        W_new = Wd - lr * g / (np.sqrt(v_new) + eps)
    elif opt == "sgd":
        W_new = Wd - lr * g
    elif opt == "sgd_momentum":
        m_new = p["momentum"] * m + g
        W_new = Wd - lr * m_new
    else:
        raise ValueError(opt)
    return W_new, m_new, v_new
