"""Pins of the oracle's contraction and of the whole step.

* dW and dX against per-element brute force with math.fsum (correctly rounded
  sums) on tiny shapes with N != K, so a transposed operand or a wrong index
  fails.
* A rank-1 closed form: dY = a u^T, X = b w^T gives dW = (a . b) u w^T.
* The tiled consume-and-discard schedule equals the two-phase schedule
  (FORGE explainer, Technical Summary section 2 "Precision and Fidelity"):
  bitwise on inputs whose sums are exact in any order, and within the float64
  summation bound on Gaussian inputs.
* Invariance of the step under a joint permutation of the tokens.
"""
import math

import numpy as np
import pytest

import synth
from oracle import numerics, optimizers, wgrad


def _fsum_wgrad(X, dY):
    T, K = X.shape
    N = dY.shape[1]
    out = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            out[n, k] = math.fsum(dY[t, n] * X[t, k] for t in range(T))
    return out


@pytest.mark.parametrize("T,N,K", [(7, 5, 3), (33, 12, 20), (64, 9, 31)])
def test_wgrad_and_dgrad_brute_force(T, N, K):
    rng = np.random.default_rng(T * 100 + N)
    X, dY, W = rng.standard_normal((T, K)), rng.standard_normal((T, N)), rng.standard_normal((N, K))
    ref = _fsum_wgrad(X, dY)
    np.testing.assert_allclose(wgrad.wgrad(X, dY), ref, rtol=1e-13, atol=1e-13)
    dx = np.array([[math.fsum(dY[t, n] * W[n, k] for n in range(N)) for k in range(K)] for t in range(T)])
    np.testing.assert_allclose(wgrad.dgrad(dY, W), dx, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(wgrad.wgrad_abs(X, dY), _fsum_wgrad(np.abs(X), np.abs(dY)), rtol=1e-13)


def test_wgrad_rank_one_closed_form():
    rng = np.random.default_rng(3)
    T, N, K = 50, 6, 11
    a, b, u, w = rng.standard_normal(T), rng.standard_normal(T), rng.standard_normal(N), rng.standard_normal(K)
    dY, X = np.outer(a, u), np.outer(b, w)
    np.testing.assert_allclose(wgrad.wgrad(X, dY), np.dot(a, b) * np.outer(u, w), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8"])
def test_integer_case_dW_is_exact(fmt):
    X, dY = synth.integer_case(1, 96, 40, 72, fmt)
    X64, dY64 = wgrad.decode_operand(X), wgrad.decode_operand(dY)
    assert np.all(np.abs(X64) <= 1) and np.all(np.abs(dY64 * 2 ** 10) <= 3)
    assert np.array_equal(X64 * 4, np.rint(X64 * 4)) and np.array_equal(dY64 * 2 ** 10, np.rint(dY64 * 2 ** 10))
    g = wgrad.wgrad(X64, dY64)
    np.testing.assert_array_equal(g, _fsum_wgrad(X64, dY64))


STEP_CASES = [("adamw", "bf16", "f32"), ("adamw", "bf16", "int8"), ("lion", "bf16", "f32"),
              ("sgd_momentum", "f32", "f32"), ("rmsprop", "bf16", "int8"), ("nadam", "bf16", "f32"),
              ("radam", "bf16", "f32"), ("adagrad", "f32", "int8"), ("sgd", "bf16", "f32")]


def _states(opt, N, K, state_fmt, rng):
    m, v = wgrad.init_states(opt, N, K, state_fmt)
    # non-zero previous moments make the check stronger than a first step
    if state_fmt == "f32":
        if m is not None:
            m = (rng.standard_normal((N, K)) * 1e-3).astype(np.float32)
        if v is not None:
            v = (np.abs(rng.standard_normal((N, K))) * 1e-6).astype(np.float32)
    else:
        if m is not None:
            m = numerics.quantize_block64(rng.standard_normal((N, K)) * 1e-3, True)
        if v is not None:
            v = numerics.quantize_block64(np.abs(rng.standard_normal((N, K))) * 1e-6, False)
    return m, v


@pytest.mark.parametrize("opt,w_fmt,state_fmt", STEP_CASES)
def test_tiled_schedule_equals_two_phase(opt, w_fmt, state_fmt):
    N, K, T = 256, 384, 64
    rng = np.random.default_rng(11)
    W = synth.random_weight(4, N, K, w_fmt)
    m, v = _states(opt, N, K, state_fmt, rng)
    h = synth.default_hyper(opt)
    # exact sums: bitwise identical
    X, dY = synth.integer_case(2, T, N, K, "bf16")
    full = wgrad.step(X, dY, W, m, v, opt, h, 3, 99, w_fmt, state_fmt)
    tiled = wgrad.step_tiled(X, dY, W, m, v, opt, h, 3, 99, w_fmt, state_fmt)
    for key in ("W", "W32", "W64", "m64", "v64"):
        if full[key] is None:
            assert tiled[key] is None
            continue
        np.testing.assert_array_equal(full[key], tiled[key], err_msg=key)
    for key in ("m", "v"):
        if full[key] is None:
            continue
        if state_fmt == "f32":
            np.testing.assert_array_equal(full[key], tiled[key])
        else:
            np.testing.assert_array_equal(full[key][0], tiled[key][0])
            np.testing.assert_array_equal(full[key][1], tiled[key][1])
    # Gaussian sums: equal within the float64 summation bound
    X, dY = synth.gaussian_case(3, T, N, K, "bf16")
    full = wgrad.step(X, dY, W, m, v, opt, h, 3, 99, w_fmt, state_fmt)
    tiled = wgrad.step_tiled(X, dY, W, m, v, opt, h, 3, 99, w_fmt, state_fmt)
    bound = T * 2.0 ** -52 * wgrad.wgrad_abs(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    assert np.all(np.abs(full["g"] - tiled["g"]) <= bound)


def test_step_invariant_under_token_permutation():
    N, K, T = 128, 256, 80
    X, dY = synth.integer_case(5, T, N, K, "bf16")
    perm = np.random.default_rng(0).permutation(T)
    Xp = synth.Operand("bf16", X.data[perm])
    dYp = synth.Operand("bf16", dY.data[perm])
    W = synth.random_weight(1, N, K, "bf16")
    m, v = wgrad.init_states("adamw", N, K, "f32")
    h = synth.default_hyper("adamw")
    a = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 5, "bf16", "f32")
    b = wgrad.step(Xp, dYp, W, m, v, "adamw", h, 1, 5, "bf16", "f32")
    for key in ("W", "m", "v", "W32"):
        np.testing.assert_array_equal(a[key], b[key])


def test_step_uses_the_full_weight_index_for_rounding_bits():
    """Each element's random bits depend on its index in the full W, so a tile of
    the weight stepped alone gets the same result as inside the full weight."""
    N, K, T = 256, 256, 32
    X, dY = synth.gaussian_case(8, T, N, K, "bf16")
    W = synth.random_weight(2, N, K, "bf16")
    h = synth.default_hyper("sgd")
    full = wgrad.step(X, dY, W, None, None, "sgd", h, 2, 7, "bf16", "f32")
    g = full["g"][128:, 128:]
    part = wgrad.apply_rule(g, W[128:, 128:], None, None, "sgd", h, 2, 7, "bf16", "f32", row0=128, col0=128, K_full=K)
    np.testing.assert_array_equal(part["W"], full["W"][128:, 128:])
    other = wgrad.apply_rule(g, W[128:, 128:], None, None, "sgd", h, 2, 7, "bf16", "f32")
    assert not np.array_equal(other["W"], full["W"][128:, 128:])


def test_int8_step_uses_fresh_fp32_moments_for_the_update():
    """Only storage is quantised: W's update uses this step's unquantised moments."""
    N, K, T = 128, 128, 16
    X, dY = synth.gaussian_case(9, T, N, K, "bf16")
    W = synth.random_weight(3, N, K, "f32")
    h = synth.default_hyper("adamw")
    m, v = wgrad.init_states("adamw", N, K, "int8")
    a = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 1, "f32", "int8")
    m0, v0 = wgrad.init_states("adamw", N, K, "f32")
    b = wgrad.step(X, dY, W, m0, v0, "adamw", h, 1, 1, "f32", "f32")
    np.testing.assert_array_equal(a["W64"], b["W64"])
    back = numerics.dequantize_block64(*a["m"], True)
    assert np.max(np.abs(back - a["m64"])) > 0       # the stored moment is quantised
