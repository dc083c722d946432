"""The GPU parity acceptance rules, checked on the CPU: the oracle's own results pass them,
results with a planted mistake (in a copy of the oracle's output) fail them."""
import numpy as np
import pytest

import synth
from oracle import numerics, optimizers, wgrad
from tests import parity as P


def _case(opt, w_fmt, state_fmt, gaussian):
    N, K, T = 128, 256, 96
    rng = np.random.default_rng(1)
    W = synth.random_weight(2, N, K, w_fmt)
    m, v = wgrad.init_states(opt, N, K, state_fmt)
    X, dY = (synth.gaussian_case if gaussian else synth.integer_case)(3, T, N, K, "bf16")
    h = synth.default_hyper(opt)
    ref = wgrad.step(X, dY, W, m, v, opt, h, 2, 11, w_fmt, state_fmt)
    env = P.envelope(opt, h, 2, ref["g"], P.grad_bound(X, dY), W, m, v, w_fmt, state_fmt) if gaussian else None
    return W, ref, env, rng


@pytest.mark.parametrize("opt", ["adamw", "lion", "sgd_momentum", "rmsprop"])
@pytest.mark.parametrize("gaussian", [False, True])
def test_oracle_result_passes_and_planted_errors_fail(opt, gaussian):
    W, ref, env, rng = _case(opt, "bf16", "f32", gaussian)
    lo, hi, mom = env if env else (None, None, {})
    slack = P.arith_slack(W, "bf16", ref["W64"])
    P.weight_close(ref["W"], ref, "bf16", lo, hi, slack=slack)
    if ref["m64"] is not None:
        P.moment_close(ref["m"], ref["m64"], "m", *mom.get("m", (None, None)))
    # one weight two ULPs off, away from any sign ambiguity
    bad = ref["W"].copy()
    i = int(np.argmax(np.abs(numerics.bf16_to_f64(bad))))
    bad.flat[i] = bad.flat[i] + 2
    with pytest.raises(AssertionError):
        P.weight_close(bad, ref, "bf16", lo, hi, slack=slack)
    if ref["m64"] is not None:
        mb = ref["m"].copy()
        j = int(np.argmax(np.abs(mb)))
        mb.flat[j] *= 1.001
        with pytest.raises(AssertionError):
            P.moment_close(mb, ref["m64"], "m", *mom.get("m", (None, None)))


def test_int8_state_check():
    _, ref, _, _ = _case("adamw", "bf16", "int8", False)
    P.int8_state_close(ref["m"], ref["m"], "m")
    codes, scales = ref["m"]
    c2 = codes.copy()
    c2.flat[5] = np.int8(np.clip(int(c2.flat[5]) + 2, -127, 127)) if abs(int(c2.flat[5])) < 120 else c2.flat[5] - 2
    with pytest.raises(AssertionError):
        P.int8_state_close((c2, scales), ref["m"], "m")


def test_ulp_helpers():
    a = numerics.bf16_rne(np.array([1.0, -1.0, 0.02, 1e-30], np.float32))
    assert np.all(P.ulp_distance(a, a) == 0)
    assert np.all(P.ulp_distance(a, a + 1) == 1)
    np.testing.assert_allclose(P.bf16_ulp(a[:3]), [2 ** -7, 2 ** -7, 2 ** -13])


@pytest.mark.parametrize("gaussian", [False, True])
def test_int8_envelope_check(gaussian):
    W, ref, env, _ = _case("adamw", "bf16", "int8", gaussian)
    mom = env[2] if env else {"m": (ref["m64"], ref["m64"]), "v": (ref["v64"], ref["v64"])}
    P.int8_envelope_close(ref["m"], *mom["m"], True, "m")
    P.int8_envelope_close(ref["v"], *mom["v"], False, "v")
    codes, scales = ref["m"]
    j = int(np.argmax(np.abs(codes.astype(int))))          # a large code, two steps off
    c2 = codes.copy()
    c2.flat[j] = np.int8(int(c2.flat[j]) - 2 * np.sign(int(c2.flat[j])))
    with pytest.raises(AssertionError):
        P.int8_envelope_close((c2, scales), *mom["m"], True, "m")
    s2 = scales.copy()
    s2.flat[3] *= 1.01                                       # a block scale 1 % off
    with pytest.raises(AssertionError):
        P.int8_envelope_close((codes, s2), *mom["m"], True, "m")


def test_dx_check():
    """The oracle's own bf16 dX passes; one element 4 ULP off (at the largest value) fails."""
    _, dY = synth.gaussian_case(82, 200, 256, 128, "bf16")
    W = synth.random_weight(83, 256, 384, "bf16")
    dY64, W64 = wgrad.decode_operand(dY), numerics.bf16_to_f64(W)
    ref = wgrad.dgrad_bf16(dY64, W64)
    P.dx_close(ref, dY64, W64)
    bad = ref.copy()
    i = int(np.argmax(np.abs(numerics.bf16_to_f64(bad))))
    bad.flat[i] = bad.flat[i] + 4
    with pytest.raises(AssertionError):
        P.dx_close(bad, dY64, W64)


@pytest.mark.parametrize("opt", ["adamw", "nadam", "radam", "rmsprop"])
@pytest.mark.parametrize("t", [2, 7])
def test_envelope_holds_every_gradient_in_the_range(opt, t):
    """From non-zero moments the Adam family's new weight has interior extrema in g'; the
    envelope's candidates must bound the oracle's value at every g' of the range.  Checked by
    brute force on a 4001-point grid per element, over moments that put the extremum inside
    the range, including tiny v, where eps shapes a narrow peak near zero."""
    rng = np.random.default_rng(5 + t)
    n = 3000
    h = synth.default_hyper(opt)
    W = synth.random_weight(6, 1, n, "bf16")[0]
    g = rng.standard_normal(n) * 10.0 ** rng.uniform(-9, -3, n)
    tau = np.abs(rng.standard_normal(n)) * 10.0 ** rng.uniform(-9, -3, n)
    m = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, -3, n)).astype(np.float32)
    v = (np.abs(rng.standard_normal(n)) * 10.0 ** rng.uniform(-20, -6, n)).astype(np.float32)
    v[::7] = 0.0
    mm = None if opt == "rmsprop" else m
    lo, hi, _ = P.envelope(opt, h, t, g, tau, W, mm, v, "bf16", "f32")
    W64 = numerics.bf16_to_f64(W)
    # slack: 1e-9 of the width, and a few fp64 rounding steps of the values themselves
    slack = 1e-9 * (hi - lo) + 32 * 2.0 ** -52 * np.maximum(np.abs(lo), np.abs(hi))
    worst = 0.0
    for f in np.linspace(-1.0, 1.0, 4001):
        w = optimizers.update(opt, h, t, g + f * tau, W64, None if mm is None else mm.astype(np.float64),
                              v.astype(np.float64))[0]
        worst = max(worst, float(np.max(np.maximum(w - hi, lo - w) / slack)))
    assert worst <= 1.0, f"a grid value lies outside the envelope by {worst:.3e} slacks"
    # the grid-and-zoom search agrees with the candidates
    lo2, hi2, _ = P.envelope(opt, h, t, g, tau, W, mm, v, "bf16", "f32", dense=True)
    assert np.max((hi2 - hi) / slack) <= 1.0 and np.max((lo - lo2) / slack) <= 1.0
