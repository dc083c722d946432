"""Pins of the oracle's eight update rules.

Library pins: torch.optim (AdamW, Adam with L2 decay, NAdam, RAdam, RMSprop,
Adagrad, SGD, SGD with momentum) run in float64 on the CPU on the same
gradients.  Lion has no torch.optim counterpart; it is pinned by closed forms.
Closed forms under constant gradients and special hyper-parameters pin the
bias corrections, the momentum sums and the RAdam branch point.
"""
import math

import numpy as np
import pytest
import torch

from oracle import optimizers
from synth import Hyper

f32 = optimizers.f32


def _run_oracle(opt, h, grads, W0):
    W = W0.copy()
    st = optimizers.STATES[opt]
    m = np.zeros_like(W0) if "m" in st else None
    v = np.zeros_like(W0) if "v" in st else None
    traj = []
    for t, g in enumerate(grads, start=1):
        W, m2, v2 = optimizers.update(opt, h, t, g, W, m, v)
        m = m2 if m2 is not None else m
        v = v2 if v2 is not None else v
        traj.append((W.copy(), None if m is None else m.copy(), None if v is None else v.copy()))
    return traj


def _torch_opt(opt, h, p):
    lr, b1, b2, eps, wd = f32(h.lr), f32(h.beta1), f32(h.beta2), f32(h.eps), f32(h.weight_decay)
    dec = optimizers.decoupled(opt, h.wd_mode)
    if opt == "adamw":
        if dec:
            return torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
        return torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    if opt == "nadam":
        return torch.optim.NAdam([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                 momentum_decay=f32(h.momentum_decay), decoupled_weight_decay=dec, foreach=False)
    if opt == "radam":
        return torch.optim.RAdam([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                 decoupled_weight_decay=dec, foreach=False)
    if opt == "rmsprop":
        assert not dec or wd == 0
        return torch.optim.RMSprop([p], lr=lr, alpha=f32(h.alpha), eps=eps, weight_decay=wd, foreach=False)
    if opt == "adagrad":
        assert not dec or wd == 0
        return torch.optim.Adagrad([p], lr=lr, eps=eps, weight_decay=wd, foreach=False)
    if opt == "sgd":
        return torch.optim.SGD([p], lr=lr, weight_decay=wd, foreach=False)
    if opt == "sgd_momentum":
        return torch.optim.SGD([p], lr=lr, momentum=f32(h.momentum), weight_decay=wd, foreach=False)
    raise ValueError(opt)


@pytest.fixture
def float64_default():
    """torch.optim keeps scalar state (step, NAdam's momentum product) in the default dtype."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


CASES = [
    ("adamw", Hyper(lr=1e-3, weight_decay=0.01)),
    ("adamw", Hyper(lr=2e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1, wd_mode=2)),
    ("nadam", Hyper(lr=1e-3)),
    ("nadam", Hyper(lr=1e-3, weight_decay=0.05)),
    ("nadam", Hyper(lr=1e-3, weight_decay=0.05, wd_mode=1)),
    ("radam", Hyper(lr=1e-3)),
    ("radam", Hyper(lr=1e-3, weight_decay=0.05)),
    ("radam", Hyper(lr=1e-3, weight_decay=0.05, wd_mode=1)),
    ("rmsprop", Hyper(lr=1e-3, alpha=0.99, eps=1e-8)),
    ("rmsprop", Hyper(lr=1e-3, alpha=0.9, eps=1e-8, weight_decay=0.02)),
    ("adagrad", Hyper(lr=1e-2, eps=1e-10)),
    ("adagrad", Hyper(lr=1e-2, eps=1e-10, weight_decay=0.02)),
    ("sgd", Hyper(lr=1e-2)),
    ("sgd", Hyper(lr=1e-2, weight_decay=0.1)),
    ("sgd_momentum", Hyper(lr=1e-2, momentum=0.9)),
    ("sgd_momentum", Hyper(lr=1e-2, momentum=0.5, weight_decay=0.1)),
]


@pytest.mark.parametrize("opt,h", CASES, ids=[f"{o}-{i}" for i, (o, _) in enumerate(CASES)])
def test_rule_matches_torch_optim_float64(opt, h, float64_default):
    rng = np.random.default_rng(hash(opt) % 1000)
    W0 = rng.standard_normal((16, 24)) * 0.02
    grads = [rng.standard_normal((16, 24)) * 0.05 * (1 + t % 3) for t in range(12)]
    ours = _run_oracle(opt, h, grads, W0)
    p = torch.nn.Parameter(torch.from_numpy(W0.copy()))
    o = _torch_opt(opt, h, p)
    for t, g in enumerate(grads):
        p.grad = torch.from_numpy(g.copy())
        o.step()
        W, m, v = ours[t]
        np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-10, atol=1e-15, err_msg=f"{opt} step {t+1}")
        state = o.state[p]
        if opt in ("adamw", "nadam", "radam"):
            np.testing.assert_allclose(m, state["exp_avg"].numpy(), rtol=1e-10, atol=1e-18)
            np.testing.assert_allclose(v, state["exp_avg_sq"].numpy(), rtol=1e-10, atol=1e-18)
        if opt == "nadam":
            s = optimizers.step_scalars(opt, h, t + 1)
            assert math.isclose(s["prod"], float(state["mu_product"]), rel_tol=1e-14)
        if opt == "rmsprop":
            np.testing.assert_allclose(v, state["square_avg"].numpy(), rtol=1e-10, atol=1e-18)
        if opt == "adagrad":
            np.testing.assert_allclose(v, state["sum"].numpy(), rtol=1e-10, atol=1e-18)
        if opt == "sgd_momentum":
            np.testing.assert_allclose(m, state["momentum_buffer"].numpy(), rtol=1e-10, atol=1e-18)


def test_radam_branch_point():
    h = Hyper(beta2=0.999)
    rho = [optimizers.step_scalars("radam", h, t)["rho_t"] for t in range(1, 8)]
    assert all(r <= 5.0 for r in rho[:5]) and all(r > 5.0 for r in rho[5:])
    assert abs(rho[4] - 4.996) < 1e-3 and abs(rho[5] - 5.994) < 1e-3
    # unrectified steps are plain momentum SGD on the bias-corrected mean
    g = np.array([0.3, -0.2])
    W, m, _ = optimizers.update("radam", h, 1, g, np.zeros(2), np.zeros(2), np.zeros(2))
    np.testing.assert_allclose(W, -f32(h.lr) * g, rtol=1e-12)


def test_adamw_constant_gradient_closed_form():
    h = Hyper(lr=1e-3, weight_decay=0.0)
    g = np.array([0.5, -0.03, 2e-7, -4.0])
    traj = _run_oracle("adamw", h, [g] * 20, np.zeros(4))
    lr, eps = f32(h.lr), f32(h.eps)
    for t, (W, m, v) in enumerate(traj, start=1):
        np.testing.assert_allclose(W, -t * lr * g / (np.abs(g) + eps), rtol=1e-10)
        np.testing.assert_allclose(m, (1 - f32(0.9) ** t) * g, rtol=1e-12)
        np.testing.assert_allclose(v, (1 - f32(0.999) ** t) * g * g, rtol=1e-12)


def test_adamw_zero_gradient_is_pure_decay_and_betas_zero_is_sign_step():
    h = Hyper(lr=1e-2, weight_decay=0.1)
    W0 = np.array([1.0, -2.0, 0.5])
    traj = _run_oracle("adamw", h, [np.zeros(3)] * 5, W0)
    for t, (W, _, _) in enumerate(traj, start=1):
        np.testing.assert_allclose(W, W0 * (1 - f32(1e-2) * f32(0.1)) ** t, rtol=1e-13)
    h0 = Hyper(lr=1e-2, beta1=0.0, beta2=0.0, weight_decay=0.0)
    g = np.array([3.0, -1e-3])
    for t in (1, 4):
        W, _, _ = optimizers.update("adamw", h0, t, g, np.zeros(2), np.full(2, 9.0), np.full(2, 9.0))
        np.testing.assert_allclose(W, -f32(1e-2) * g / (np.abs(g) + f32(1e-8)), rtol=1e-12)


def test_lion_closed_forms():
    h = Hyper(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01)
    lr, wd, b1, b2 = f32(h.lr), f32(h.weight_decay), f32(h.beta1), f32(h.beta2)
    W0 = np.array([0.02, -0.01, 0.005, 0.0])
    g = np.array([0.3, -0.7, 0.0, 1e-9])
    W, m, v = optimizers.update("lion", h, 1, g, W0, np.zeros(4), None)
    np.testing.assert_allclose(W, W0 - lr * (np.sign(g) + wd * W0), rtol=1e-14, atol=1e-20)
    np.testing.assert_allclose(m, (1 - b2) * g, rtol=1e-14)
    assert v is None
    # constant gradient, no decay: every step moves by lr against the sign of g
    h0 = Hyper(lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.0)
    traj = _run_oracle("lion", h0, [g] * 7, W0)
    for t, (Wt, mt, _) in enumerate(traj, start=1):
        np.testing.assert_allclose(Wt, W0 - t * lr * np.sign(g), rtol=1e-13, atol=1e-20)
        np.testing.assert_allclose(mt, (1 - b2 ** t) * g, rtol=1e-12)
    # the interpolation inside sign() uses beta1, the moment update uses beta2
    W, m, _ = optimizers.update("lion", h0, 3, np.array([-20.0, -5.0]), np.zeros(2), np.ones(2), None)
    np.testing.assert_allclose(W, [lr, -lr], rtol=1e-14)        # c = 0.9 - 2 < 0 ; c = 0.9 - 0.5 > 0
    np.testing.assert_allclose(m, b2 * 1.0 + (1 - b2) * np.array([-20.0, -5.0]), rtol=1e-14)
    # zero gradient with decay: pure decay
    traj = _run_oracle("lion", h, [np.zeros(4)] * 3, W0)
    np.testing.assert_allclose(traj[-1][0], W0 * (1 - lr * wd) ** 3, rtol=1e-13)


def test_sgd_family_and_adaptive_closed_forms():
    g = np.array([0.4, -1.5, 1e-3])
    h = Hyper(lr=1e-2, momentum=0.9)
    lr, mu = f32(h.lr), f32(h.momentum)
    sgd = _run_oracle("sgd", h, [g] * 6, np.zeros(3))
    sgdm = _run_oracle("sgd_momentum", h, [g] * 6, np.zeros(3))
    for t in range(1, 7):
        np.testing.assert_allclose(sgd[t - 1][0], -t * lr * g, rtol=1e-13)
        coef = sum((1 - mu ** i) / (1 - mu) for i in range(1, t + 1))
        np.testing.assert_allclose(sgdm[t - 1][0], -lr * g * coef, rtol=1e-12)
        np.testing.assert_allclose(sgdm[t - 1][1], g * (1 - mu ** t) / (1 - mu), rtol=1e-12)
    # momentum 0 is plain SGD, also with coupled decay
    h0 = Hyper(lr=1e-2, momentum=0.0, weight_decay=0.3)
    rng = np.random.default_rng(5)
    grads = [rng.standard_normal(5) for _ in range(4)]
    W0 = rng.standard_normal(5)
    a = _run_oracle("sgd", h0, grads, W0)
    b = _run_oracle("sgd_momentum", h0, grads, W0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x[0], y[0])
    # AdaGrad: accumulator t g^2 ; RMSprop: v_t = (1 - alpha^t) g^2
    ha = Hyper(lr=1e-2, eps=1e-10)
    tr = _run_oracle("adagrad", ha, [g] * 5, np.zeros(3))
    W = np.zeros(3)
    for t in range(1, 6):
        W = W - f32(1e-2) * g / (np.sqrt(t) * np.abs(g) + f32(1e-10))
        np.testing.assert_allclose(tr[t - 1][0], W, rtol=1e-12)
        np.testing.assert_allclose(tr[t - 1][2], t * g * g, rtol=1e-13)
    hr = Hyper(lr=1e-3, alpha=0.99, eps=1e-8)
    tr = _run_oracle("rmsprop", hr, [g] * 5, np.zeros(3))
    for t in range(1, 6):
        np.testing.assert_allclose(tr[t - 1][2], (1 - f32(0.99) ** t) * g * g, rtol=1e-12)
    W1 = tr[0][0]
    np.testing.assert_allclose(W1, -f32(1e-3) * g / (np.sqrt(1 - f32(0.99)) * np.abs(g) + f32(1e-8)), rtol=1e-12)


def test_nadam_step_one_closed_form():
    h = Hyper(lr=1e-3)
    b1, psi, lr, eps = f32(0.9), f32(0.004), f32(1e-3), f32(1e-8)
    mu1 = b1 * (1 - 0.5 * 0.96 ** psi)
    mu2 = b1 * (1 - 0.5 * 0.96 ** (2 * psi))
    g = np.array([0.2, -3.0])
    W, m, v = optimizers.update("nadam", h, 1, g, np.zeros(2), np.zeros(2), np.zeros(2))
    # at t = 1 the bias-corrected second moment is g^2 and m = (1 - beta1) g
    want = -lr * g / (np.abs(g) + eps) * (1.0 + mu2 * (1 - b1) / (1 - mu1 * mu2))
    np.testing.assert_allclose(W, want, rtol=1e-12)


def test_step_count_must_start_at_one():
    with pytest.raises(ValueError):
        optimizers.step_scalars("adamw", Hyper(), 0)
