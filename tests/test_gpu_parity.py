"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case prints what identifies it before touching the GPU.  Shapes span several 128 x 128
tiles and a ragged final token slab (T = 200 is not a multiple of the 32 / 64 / 128-token
slabs of the fp32 / bf16 / fp8 mainloops).

Protocols (see tests/parity.py for the acceptance rules):
  * exact-sum inputs, oracle-fed: before each step the device state is set to the oracle's
    stored state after the previous step, so each step is compared on identical inputs;
  * exact-sum inputs, free-running: the device keeps its own state for several steps;
  * Gaussian inputs with the workloads' standard deviations: the envelope over the fp32
    summation error bound of the gradient.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import numerics, optimizers, wgrad
from tests import parity as P

pytestmark = pytest.mark.gpu

N, K, T = 256, 384, 200


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    if not __import__("os").path.exists(forge.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def _init_states(opt, state_fmt, rng, N=N, K=K):
    return P.init_states(opt, state_fmt, rng, N, K)


_compare = P.compare


EXACT = [(opt, i, w, s) for opt in synth.OPTIMIZERS
         for (i, w) in (("bf16", "bf16"), ("f32", "f32"), ("fp8", "bf16"), ("bf16", "f32"))
         for s in ("f32", "int8")]


@pytest.mark.parametrize("opt,in_fmt,w_fmt,state_fmt", EXACT, ids=["-".join(c) for c in EXACT])
def test_fused_step_exact_inputs_oracle_fed(lib, opt, in_fmt, w_fmt, state_fmt):
    rng = np.random.default_rng(abs(hash((opt, in_fmt, w_fmt, state_fmt))) % 2 ** 32)
    h = synth.default_hyper(opt)
    seed = 1234 + synth.OPTIMIZERS.index(opt)
    W = synth.random_weight(7, N, K, w_fmt)
    m, v = _init_states(opt, state_fmt, rng)
    for i, t in enumerate((1, 2, 7)):
        _say("exact oracle-fed", opt, in_fmt, w_fmt, state_fmt, "step", t)
        X, dY = synth.integer_case(100 * i + 3, T, N, K, in_fmt)
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, seed, w_fmt, state_fmt)
        d = P.DeviceStep(W, m, v, w_fmt, state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, seed, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), w_fmt, state_fmt, W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


FREE = [("adamw", "bf16", "bf16"), ("lion", "bf16", "bf16"), ("nadam", "fp8", "bf16"), ("sgd_momentum", "f32", "f32"),
        ("radam", "bf16", "bf16"), ("rmsprop", "bf16", "f32"), ("adagrad", "bf16", "bf16"), ("sgd", "fp8", "bf16")]


@pytest.mark.parametrize("opt,in_fmt,w_fmt", FREE, ids=["-".join(c) for c in FREE])
def test_fused_free_running_exact_inputs(lib, opt, in_fmt, w_fmt):
    """The device keeps its own W, m, v over 7 steps (fp32 moments)."""
    h = synth.default_hyper(opt)
    W = synth.random_weight(9, N, K, w_fmt)
    m, v = wgrad.init_states(opt, N, K, "f32")
    d = P.DeviceStep(W, m, v, w_fmt, "f32")
    carried = 0.0
    for t in range(1, 8):
        _say("exact free-running", opt, in_fmt, w_fmt, "step", t)
        X, dY = synth.integer_case(500 + t, T, N, K, in_fmt)
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 77, w_fmt, "f32")
        d.fused(lib, X, dY, opt, h, t, 77)
        gW, gm, gv = d.host()
        # The device carries its own weight.  A difference left by an earlier step (one rounding
        # of a weight that then moves to a smaller binade can be several ULPs of the new one)
        # carries over; each step may add one ULP (stochastic-rounding threshold) plus the fp32
        # rounding of the rule's arithmetic.
        slack = P.arith_slack(W, w_fmt, ref["W64"])
        if w_fmt == "bf16":
            x, r = numerics.bf16_to_f64(gW), numerics.bf16_to_f64(ref["W"])
            allowed = carried * (1 + 1e-6) + P.bf16_ulp(ref["W"]) * (1 + 1e-6) + slack
        else:
            x, r = gW.astype(np.float64), ref["W"].astype(np.float64)
            allowed = carried * (1 + 1e-6) + 1e-6 + 1e-4 * np.abs(r) + slack
        diff = np.abs(x - r)
        bad = diff > allowed
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise AssertionError(f"step {t}: {int(bad.sum())} weights off; first got {x.flat[i]:.8e} want "
                                 f"{r.flat[i]:.8e} (allowed {allowed.flat[i]:.3e}, carried {np.asarray(carried + 0 * x).flat[i]:.3e})")
        carried = diff
        P.state_close(gm, ref["m"], ref["m64"], "f32", f"step {t} m")
        P.state_close(gv, ref["v"], ref["v64"], "f32", f"step {t} v")
        W, m, v = ref["W"], ref["m"], ref["v"]


GAUSS = ([(opt, "bf16", "bf16", "f32") for opt in synth.OPTIMIZERS]
         + [("adamw", "bf16", "bf16", "int8"), ("adamw", "fp8", "bf16", "f32"), ("lion", "fp8", "bf16", "f32"),
            ("adamw", "f32", "f32", "f32"), ("rmsprop", "bf16", "bf16", "int8")])


@pytest.mark.parametrize("opt,in_fmt,w_fmt,state_fmt", GAUSS, ids=["-".join(c) for c in GAUSS])
def test_fused_step_gaussian_envelope(lib, opt, in_fmt, w_fmt, state_fmt):
    rng = np.random.default_rng(5)
    h = synth.default_hyper(opt)
    W = synth.random_weight(11, N, K, w_fmt)
    m, v = _init_states(opt, state_fmt, rng)
    for i, t in enumerate((1, 3, 6)):
        _say("gaussian envelope", opt, in_fmt, w_fmt, state_fmt, "step", t)
        X, dY = synth.gaussian_case(40 + i, T, N, K, in_fmt)
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 99, w_fmt, state_fmt)
        tau = P.grad_bound(X, dY)
        env = P.envelope(opt, h, t, ref["g"], tau, W, m, v, w_fmt, state_fmt)
        d = P.DeviceStep(W, m, v, w_fmt, state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, 99, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), w_fmt, state_fmt, W, env, tag=f"step {t}")
        W, m, v = ref["W"], ref["m"], ref["v"]


UNF = [(opt, "bf16", "bf16", "f32") for opt in synth.OPTIMIZERS] + [
    ("adamw", "bf16", "bf16", "int8"), ("adamw", "fp8", "bf16", "f32"), ("adamw", "f32", "f32", "f32"),
    ("lion", "bf16", "f32", "int8")]


@pytest.mark.parametrize("opt,in_fmt,w_fmt,state_fmt", UNF, ids=["-".join(c) for c in UNF])
def test_fused_equals_unfused_bitwise(lib, opt, in_fmt, w_fmt, state_fmt):
    """Same contraction, same rule code: the two schedules give identical bits (exactness claim)."""
    _say("fused vs unfused", opt, in_fmt, w_fmt, state_fmt)
    rng = np.random.default_rng(8)
    h = synth.default_hyper(opt)
    W = synth.random_weight(12, N, K, w_fmt)
    m, v = _init_states(opt, state_fmt, rng)
    X, dY = synth.gaussian_case(60, T, N, K, in_fmt)
    a = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    b = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    pa = a.fused(lib, X, dY, opt, h, 4, 5, preround=True)
    pb, dW = b.unfused(lib, X, dY, opt, h, 4, 5, preround=True)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)
    for x, y in zip(a.host(), b.host()):
        if x is None:
            assert y is None
        elif isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        else:
            assert np.array_equal(x, y)


@pytest.mark.parametrize("in_fmt", ["bf16", "f32", "fp8"])
def test_wgrad_gemm_matches_oracle(lib, in_fmt):
    _say("wgrad gemm", in_fmt)
    X, dY = synth.integer_case(70, T, N, K, in_fmt)
    dW = torch.empty((N, K), dtype=torch.float32, device="cuda")
    Xd, xs = P.dev_operand(X)
    Dd, ds = P.dev_operand(dY)
    lib.wgrad_gemm(Xd, Dd, dW, x_scale=xs, dy_scale=ds)
    ref = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    np.testing.assert_array_equal(dW.cpu().numpy().astype(np.float64), ref)      # exact sums: bitwise
    X, dY = synth.gaussian_case(71, T, N, K, in_fmt)
    Xd, xs = P.dev_operand(X)
    Dd, ds = P.dev_operand(dY)
    lib.wgrad_gemm(Xd, Dd, dW, x_scale=xs, dy_scale=ds)
    ref = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    err = np.abs(dW.cpu().numpy().astype(np.float64) - ref)
    tau = P.grad_bound(X, dY)
    assert np.all(err <= tau), float(np.max(err / np.maximum(tau, 1e-300)))
    print(f"  max |err| / bound = {float(np.max(err / np.maximum(tau, 1e-300))):.3e}")


# fp32 inputs take 64 x 64 tiles while a weight has fewer 128 x 128 tiles than the device has
# CUs (256 x 384 above), and 128 x 128 tiles from there on (2048 x 2048: 256 tiles).
F32_128 = [("adamw", "f32"), ("lion", "int8"), ("nadam", "int8dyn"), ("sgd_momentum", "f32")]


@pytest.mark.parametrize("opt,state_fmt", F32_128, ids=["-".join(c) for c in F32_128])
def test_f32_large_tiles_exact_oracle_fed(lib, opt, state_fmt):
    Nn = Kn = 2048
    rng = np.random.default_rng(91)
    h = synth.default_hyper(opt)
    W = synth.random_weight(92, Nn, Kn, "f32")
    m, v = _init_states(opt, state_fmt, rng, Nn, Kn)
    for i, t in enumerate((1, 3)):
        _say("f32 128x128 tiles exact oracle-fed", opt, state_fmt, Nn, Kn, "step", t)
        X, dY = synth.integer_case(390 + i, T, Nn, Kn, "f32")
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 23, "f32", state_fmt)
        d = P.DeviceStep(W, m, v, "f32", state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, 23, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), "f32", state_fmt, W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


def test_f32_large_tiles_wgrad_gemm_exact(lib):
    Nn = Kn = 2048
    _say("wgrad gemm f32 128x128 tiles", Nn, Kn)
    X, dY = synth.integer_case(395, T, Nn, Kn, "f32")
    dW = torch.empty((Nn, Kn), dtype=torch.float32, device="cuda")
    Xd, xs = P.dev_operand(X)
    Dd, ds = P.dev_operand(dY)
    lib.wgrad_gemm(Xd, Dd, dW, x_scale=xs, dy_scale=ds)
    ref = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    np.testing.assert_array_equal(dW.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("Tn,Nn,Kn", [(200, 256, 384), (128, 384, 256), (1, 128, 128), (333, 640, 128)])
def test_dgrad_matches_oracle(lib, Tn, Nn, Kn):
    _say("dgrad", Tn, Nn, Kn)
    # exact sums: dY and W on a dyadic grid
    _, dY = synth.integer_case(80, Tn, Nn, 128, "bf16")
    Wi, _ = synth.integer_case(81, Nn, 128, Kn, "bf16")      # X-shaped [Nn, Kn] grid values in [-1, 1]
    Wd = P.dev_weight(Wi.data, "bf16")
    dYd, _ = P.dev_operand(dY)
    dX = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    lib.dgrad(dYd, Wd, dX)
    ref = wgrad.dgrad_bf16(wgrad.decode_operand(dY), numerics.bf16_to_f64(Wi.data))
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # Gaussian: bf16 nearest-even of an fp32 sum in the kernel's order, within the summation
    # bound of the exact product plus one ULP
    _, dY = synth.gaussian_case(82, Tn, Nn, 128, "bf16")
    W = synth.random_weight(83, Nn, Kn, "bf16")
    dYd, _ = P.dev_operand(dY)
    lib.dgrad(dYd, P.dev_weight(W, "bf16"), dX)
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    P.dx_close(got, wgrad.decode_operand(dY), numerics.bf16_to_f64(W))


# 256-token x 256-column dX tiles in one 8-wave workgroup per CU are used when K % 256 == 0 and
# there are at least as many of them as CUs (256 on an MI355X): 4196 x 4096 is 17 x 16 = 272
# tiles with a ragged last token block, 2048 x 8192 is 8 x 32 = 256.  4196 x 4224 (K / 128 odd)
# stays on the 256 x 128 tiles.  Same two checks as above: exact sums bitwise, Gaussian within
# the summation bound.
@pytest.mark.parametrize("Tn,Nn,Kn", [(4196, 256, 4096), (2048, 384, 8192), (4196, 256, 4224)])
def test_dgrad_wide_tiles_match_oracle(lib, Tn, Nn, Kn):
    _say("dgrad wide", Tn, Nn, Kn)
    _, dY = synth.integer_case(90, Tn, Nn, 128, "bf16")
    Wi, _ = synth.integer_case(91, Nn, 128, Kn, "bf16")
    dYd, _ = P.dev_operand(dY)
    dX = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    lib.dgrad(dYd, P.dev_weight(Wi.data, "bf16"), dX)
    ref = wgrad.dgrad_bf16(wgrad.decode_operand(dY), numerics.bf16_to_f64(Wi.data))
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    _, dY = synth.gaussian_case(92, Tn, Nn, 128, "bf16")
    W = synth.random_weight(93, Nn, Kn, "bf16")
    dYd, _ = P.dev_operand(dY)
    lib.dgrad(dYd, P.dev_weight(W, "bf16"), dX)
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    P.dx_close(got, wgrad.decode_operand(dY), numerics.bf16_to_f64(W))


def test_backward_step_reads_the_old_weight(lib):
    """dX must see W before the update (limitation stated in the explainer's section 5)."""
    _say("ordering")
    X, dY = synth.gaussian_case(90, T, N, K, "bf16")
    W = synth.random_weight(91, N, K, "bf16")
    m, v = wgrad.init_states("adamw", N, K, "f32")
    h = synth.Hyper(lr=0.05, weight_decay=0.0)   # large steps make the order visible
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    Xd, _ = P.dev_operand(X)
    dYd, _ = P.dev_operand(dY)
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    lib.linear_backward_step(Xd, dYd, d.W, dX, d.m, d.v, opt="adamw", hyper=h, step=1, seed=3)
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    dY64 = wgrad.decode_operand(dY)
    P.dx_close(got, dY64, numerics.bf16_to_f64(W), "dX from the old weight")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 3, "bf16", "f32")
    with pytest.raises(AssertionError):                 # the reversed order is visibly different
        P.dx_close(got, dY64, numerics.bf16_to_f64(ref["W"]), "dX from the new weight")
    lo, hi, _ = P.envelope("adamw", h, 1, ref["g"], P.grad_bound(X, dY), W, m, v, "bf16", "f32")
    P.weight_close(d.host()[0], ref, "bf16", lo, hi, slack=P.arith_slack(W, "bf16", ref["W64"]))


@pytest.mark.parametrize("Tn", [0, 1, 64, 65])
def test_edge_token_counts(lib, Tn):
    _say("edge T", Tn)
    h = synth.default_hyper("adamw")
    X, dY = synth.integer_case(95, Tn, N, K, "bf16")
    W = synth.random_weight(96, N, K, "bf16")
    m, v = wgrad.init_states("adamw", N, K, "f32")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 4, "bf16", "f32")
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    pre = d.fused(lib, X, dY, "adamw", h, 1, 4, preround=True)
    gW, gm, gv = d.host()
    _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W)
    if Tn == 0:  # zero gradient: pure decoupled decay
        np.testing.assert_allclose(pre.cpu().numpy(), numerics.bf16_to_f64(W) * (1 - np.float32(1e-3) * np.float32(0.01)),
                                   rtol=1e-6)


def test_empty_weight_is_a_no_op(lib):
    _say("empty N")
    X = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    lib.wgrad_step(X, dY, W, torch.zeros((0, 128), device="cuda"), torch.zeros((0, 128), device="cuda"),
                   opt="adamw", hyper=synth.default_hyper("adamw"), step=1, seed=1)
    torch.cuda.synchronize()


def test_determinism_and_resume(lib):
    """Same inputs, seed and step give the same bits; 5 steps straight == 2 + host round trip + 3."""
    _say("determinism / resume")
    h = synth.default_hyper("adamw")
    W0 = synth.random_weight(20, N, K, "bf16")
    m0, v0 = wgrad.init_states("adamw", N, K, "f32")
    ins = [synth.gaussian_case(200 + t, T, N, K, "bf16") for t in range(1, 6)]
    a = P.DeviceStep(W0, m0, v0, "bf16", "f32")
    for t in range(1, 6):
        a.fused(lib, *ins[t - 1], "adamw", h, t, 42)
    b = P.DeviceStep(W0, m0, v0, "bf16", "f32")
    for t in range(1, 3):
        b.fused(lib, *ins[t - 1], "adamw", h, t, 42)
    Wb, mb, vb = b.host()
    c = P.DeviceStep(Wb, mb, vb, "bf16", "f32")
    for t in range(3, 6):
        c.fused(lib, *ins[t - 1], "adamw", h, t, 42)
    for x, y in zip(a.host(), c.host()):
        assert np.array_equal(x, y)
    a2 = P.DeviceStep(W0, m0, v0, "bf16", "f32")
    for t in range(1, 6):
        a2.fused(lib, *ins[t - 1], "adamw", h, t, 42)
    for x, y in zip(a.host(), a2.host()):
        assert np.array_equal(x, y)


def test_stochastic_rounding_escapes_the_dead_zone(lib):
    """Sub-ULP updates: nearest-even leaves W frozen, stochastic rounding tracks the fp32 sum."""
    _say("dead zone")
    n, k, steps = 256, 256, 40
    X = torch.zeros((64, k), dtype=torch.bfloat16, device="cuda")
    X[0, :] = 1.0
    dY = torch.zeros((64, n), dtype=torch.bfloat16, device="cuda")
    dY[0, :] = 1.0                                   # g = 1 everywhere
    w0 = 0.02
    ulp = float(P.bf16_ulp(numerics.bf16_rne(np.array([w0], np.float32)))[0])
    lr = 0.1 * ulp                                   # SGD: each step moves W by 0.1 ULP
    h = synth.Hyper(lr=lr)
    W_rne = torch.full((n, k), w0, dtype=torch.bfloat16, device="cuda")
    W_sr = W_rne.clone()
    start = float(W_rne[0, 0])
    for t in range(1, steps + 1):
        lib.wgrad_step(X, dY, W_rne, opt="sgd", hyper=h, step=t, seed=5, sr=False)
        lib.wgrad_step(X, dY, W_sr, opt="sgd", hyper=h, step=t, seed=5)
    torch.cuda.synchronize()
    assert torch.all(W_rne == start)
    drift = W_sr.double().cpu().numpy() - start
    want = -steps * float(np.float32(lr))
    sd = ulp * np.sqrt(steps * 0.25) / np.sqrt(n * k)
    assert abs(drift.mean() - want) < 6 * sd + 1e-3 * abs(want), (drift.mean(), want)
    # and it equals the oracle's stream, element by element, for the first step
    Wb = numerics.bf16_rne(np.full((n, k), w0, np.float32))
    Xo = synth.Operand("bf16", X.view(torch.int16).cpu().numpy().view(np.uint16))
    Do = synth.Operand("bf16", dY.view(torch.int16).cpu().numpy().view(np.uint16))
    ref = wgrad.step(Xo, Do, Wb, None, None, "sgd", h, 1, 5, "bf16", "f32")
    Wg = P.dev_weight(Wb, "bf16")
    lib.wgrad_step(X, dY, Wg, opt="sgd", hyper=h, step=1, seed=5)
    np.testing.assert_array_equal(P.host_weight(Wg, "bf16"), ref["W"])


# ----------------------------------------------------------------------------- 256 x 128 DMA path
# bf16 inputs with N % 256 == 0 and at least 256 tiles of 256 x 128 take the LDS-DMA mainloop.
N2, K2 = 2048, 4096
V2 = [("adamw", "bf16", "f32"), ("adamw", "bf16", "int8"), ("lion", "bf16", "f32"), ("nadam", "f32", "f32"),
      ("radam", "bf16", "f32"), ("sgd_momentum", "bf16", "int8"), ("rmsprop", "f32", "f32")]


@pytest.mark.parametrize("opt,w_fmt,state_fmt", V2, ids=["-".join(c) for c in V2])
def test_v2_exact_inputs_oracle_fed(lib, opt, w_fmt, state_fmt):
    rng = np.random.default_rng(31)
    h = synth.default_hyper(opt)
    W = synth.random_weight(33, N2, K2, w_fmt)
    m, v = _init_states(opt, state_fmt, rng, N2, K2)
    for i, t in enumerate((1, 6)):
        _say("v2 exact oracle-fed", opt, w_fmt, state_fmt, "step", t)
        X, dY = synth.integer_case(300 + i, T, N2, K2, "bf16")
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 5, w_fmt, state_fmt)
        d = P.DeviceStep(W, m, v, w_fmt, state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, 5, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), w_fmt, state_fmt, W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


def test_v2_gaussian_envelope(lib):
    rng = np.random.default_rng(32)
    h = synth.default_hyper("adamw")
    W = synth.random_weight(34, N2, K2, "bf16")
    m, v = _init_states("adamw", "f32", rng, N2, K2)
    for i, t in enumerate((1, 3)):
        _say("v2 gaussian envelope step", t)
        X, dY = synth.gaussian_case(310 + i, T, N2, K2, "bf16")
        ref = wgrad.step(X, dY, W, m, v, "adamw", h, t, 6, "bf16", "f32")
        env = P.envelope("adamw", h, t, ref["g"], P.grad_bound(X, dY), W, m, v, "bf16", "f32")
        d = P.DeviceStep(W, m, v, "bf16", "f32")
        pre = d.fused(lib, X, dY, "adamw", h, t, 6, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, env, tag=f"step {t}")
        W, m, v = ref["W"], ref["m"], ref["v"]


@pytest.mark.parametrize("state_fmt", ["f32", "int8"])
def test_v2_fused_equals_unfused_bitwise(lib, state_fmt):
    _say("v2 fused vs unfused", state_fmt)
    rng = np.random.default_rng(35)
    h = synth.default_hyper("adamw")
    W = synth.random_weight(36, N2, K2, "bf16")
    m, v = _init_states("adamw", state_fmt, rng, N2, K2)
    X, dY = synth.gaussian_case(320, T, N2, K2, "bf16")
    a = P.DeviceStep(W, m, v, "bf16", state_fmt)
    b = P.DeviceStep(W, m, v, "bf16", state_fmt)
    pa = a.fused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    pb, dW = b.unfused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)
    for x, y in zip(a.host(), b.host()):
        if isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        else:
            assert np.array_equal(x, y)
    # the materialised gradient of the unfused path against the oracle
    ref = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    err = np.abs(dW.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= P.grad_bound(X, dY))


@pytest.mark.parametrize("Tn", [0, 1, 63, 64, 65, 129])
def test_v2_token_counts(lib, Tn):
    _say("v2 edge T", Tn)
    h = synth.default_hyper("adamw")
    X, dY = synth.integer_case(330 + Tn, Tn, N2, K2, "bf16")
    W = synth.random_weight(37, N2, K2, "bf16")
    m, v = wgrad.init_states("adamw", N2, K2, "f32")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 8, "bf16", "f32")
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    pre = d.fused(lib, X, dY, "adamw", h, 1, 8, preround=True)
    gW, gm, gv = d.host()
    _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, tag=f"T={Tn}")


# ----------------------------------------------------------------------------- full + half tiles
# 4096 x 4224 has 16 x 33 = 528 tiles of 256 x 128: with 512 workgroup slots the launcher keeps
# 512 full tiles and turns the last k-block column into 32 half tiles of 128 x 128 (the 2048 x
# 4096 shapes above run as half tiles only).
N3, K3 = 4096, 4224


FULL_RULES = [(opt, s) for opt in synth.OPTIMIZERS for s in ("f32", "int8")]


@pytest.mark.parametrize("opt,state_fmt", FULL_RULES, ids=["-".join(c) for c in FULL_RULES])
def test_v2_full_tiles_every_rule_exact_oracle_fed(lib, opt, state_fmt):
    """Every rule and moment format on the 256 x 128 tiles (with their two-half
    epilogue) and half tiles in one launch, exact-sum inputs, steps 1 and 6 from the oracle's
    stored state."""
    rng = np.random.default_rng(43)
    h = synth.default_hyper(opt)
    W = synth.random_weight(44, N3, K3, "bf16")
    m, v = _init_states(opt, state_fmt, rng, N3, K3)
    for i, t in enumerate((1, 6)):
        _say("v2 full tiles exact oracle-fed", opt, state_fmt, "step", t)
        X, dY = synth.integer_case(345 + i, T, N3, K3, "bf16")
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 13, "bf16", state_fmt)
        d = P.DeviceStep(W, m, v, "bf16", state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, 13, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", state_fmt, W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


@pytest.mark.parametrize("opt,state_fmt", [("adamw", "f32"), ("lion", "int8")])
def test_v2_full_and_half_tiles_exact(lib, opt, state_fmt):
    _say("v2 full + half tiles exact", opt, state_fmt)
    rng = np.random.default_rng(41)
    h = synth.default_hyper(opt)
    W = synth.random_weight(42, N3, K3, "bf16")
    m, v = _init_states(opt, state_fmt, rng, N3, K3)
    X, dY = synth.integer_case(340, T, N3, K3, "bf16")
    ref = wgrad.step(X, dY, W, m, v, opt, h, 3, 12, "bf16", state_fmt)
    d = P.DeviceStep(W, m, v, "bf16", state_fmt)
    pre = d.fused(lib, X, dY, opt, h, 3, 12, preround=True)
    gW, gm, gv = d.host()
    _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", state_fmt, W, tag="full+half",
             lion=(h, 3, m, v) if opt == "lion" else None)
    u = P.DeviceStep(W, m, v, "bf16", state_fmt)
    pu, dW = u.unfused(lib, X, dY, opt, h, 3, 12, preround=True)
    torch.cuda.synchronize()
    assert torch.equal(pre, pu)
    ref_g = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    np.testing.assert_array_equal(dW.cpu().numpy().astype(np.float64), ref_g)   # exact sums: bitwise


# ----------------------------------------------------------------------------- fp8 DMA path
# fp8 e4m3 inputs with N % 256 == 0 and at least 256 tiles of 256 x 128 take the 8-bit
# transpose-read mainloop (64-token slabs; T = 200 leaves a ragged last slab).
V8 = [("adamw", "bf16", "f32"), ("nadam", "bf16", "int8"), ("lion", "f32", "f32"), ("sgd", "bf16", "f32")]


@pytest.mark.parametrize("opt,w_fmt,state_fmt", V8, ids=["-".join(c) for c in V8])
def test_v8_exact_inputs_oracle_fed(lib, opt, w_fmt, state_fmt):
    rng = np.random.default_rng(51)
    h = synth.default_hyper(opt)
    W = synth.random_weight(52, N2, K2, w_fmt)
    m, v = _init_states(opt, state_fmt, rng, N2, K2)
    for i, t in enumerate((1, 4)):
        _say("v8 exact oracle-fed", opt, w_fmt, state_fmt, "step", t)
        X, dY = synth.integer_case(350 + i, T, N2, K2, "fp8")
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 7, w_fmt, state_fmt)
        d = P.DeviceStep(W, m, v, w_fmt, state_fmt)
        pre = d.fused(lib, X, dY, opt, h, t, 7, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), w_fmt, state_fmt, W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


def test_v8_gaussian_envelope(lib):
    rng = np.random.default_rng(53)
    h = synth.default_hyper("adamw")
    W = synth.random_weight(54, N2, K2, "bf16")
    m, v = _init_states("adamw", "f32", rng, N2, K2)
    _say("v8 gaussian envelope")
    X, dY = synth.gaussian_case(360, T, N2, K2, "fp8")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 2, 8, "bf16", "f32")
    env = P.envelope("adamw", h, 2, ref["g"], P.grad_bound(X, dY), W, m, v, "bf16", "f32")
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    pre = d.fused(lib, X, dY, "adamw", h, 2, 8, preround=True)
    gW, gm, gv = d.host()
    _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, env, tag="fp8 gaussian")


def test_v8_fused_equals_unfused_bitwise(lib):
    _say("v8 fused vs unfused")
    rng = np.random.default_rng(55)
    h = synth.default_hyper("adamw")
    W = synth.random_weight(56, N2, K2, "bf16")
    m, v = _init_states("adamw", "f32", rng, N2, K2)
    X, dY = synth.gaussian_case(361, T, N2, K2, "fp8")
    a = P.DeviceStep(W, m, v, "bf16", "f32")
    b = P.DeviceStep(W, m, v, "bf16", "f32")
    pa = a.fused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    pb, dW = b.unfused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)
    for x, y in zip(a.host(), b.host()):
        assert np.array_equal(x, y)
    ref = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    err = np.abs(dW.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= P.grad_bound(X, dY))


@pytest.mark.parametrize("Tn", [0, 1, 63, 64, 65, 129])
def test_v8_token_counts(lib, Tn):
    _say("v8 edge T", Tn)
    h = synth.default_hyper("adamw")
    X, dY = synth.integer_case(370 + Tn, Tn, N2, K2, "fp8")
    W = synth.random_weight(57, N2, K2, "bf16")
    m, v = wgrad.init_states("adamw", N2, K2, "f32")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 8, "bf16", "f32")
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    pre = d.fused(lib, X, dY, "adamw", h, 1, 8, preround=True)
    gW, gm, gv = d.host()
    _compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, tag=f"fp8 T={Tn}")


# ----------------------------------------------------------------------------- dynamic 8-bit map
# Moments in the dynamic 8-bit map (the comparison format of common 8-bit optimizers), every
# rule, on the register-staged path (256 x 384), the bf16 LDS-DMA full and half tiles
# (4096 x 4224) and the fp8 path; exact-sum inputs, steps 1 and 6 from the oracle's stored state.
# Codes are compared in value order (within one step).
DYN = ([(opt, "bf16", N, K) for opt in synth.OPTIMIZERS] + [(opt, "bf16", N3, K3) for opt in synth.OPTIMIZERS]
       + [("adamw", "fp8", N3, K3), ("lion", "fp8", N3, K3), ("rmsprop", "f32", N, K)])


@pytest.mark.parametrize("opt,in_fmt,Nn,Kn", DYN, ids=[f"{o}-{i}-{n}x{k}" for o, i, n, k in DYN])
def test_dynamic_map_exact_oracle_fed(lib, opt, in_fmt, Nn, Kn):
    if "m" not in optimizers.STATES[opt] and "v" not in optimizers.STATES[opt]:
        pytest.skip("the rule keeps no moment")
    rng = np.random.default_rng(71)
    h = synth.default_hyper(opt)
    w_fmt = "f32" if in_fmt == "f32" else "bf16"
    W = synth.random_weight(72, Nn, Kn, w_fmt)
    m, v = _init_states(opt, "int8dyn", rng, Nn, Kn)
    for i, t in enumerate((1, 6)):
        _say("dynamic map exact oracle-fed", opt, in_fmt, Nn, Kn, "step", t)
        X, dY = synth.integer_case(380 + i, T, Nn, Kn, in_fmt)
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 21, w_fmt, "int8dyn")
        d = P.DeviceStep(W, m, v, w_fmt, "int8dyn")
        pre = d.fused(lib, X, dY, opt, h, t, 21, preround=True)
        gW, gm, gv = d.host()
        _compare(ref, gW, gm, gv, pre.cpu().numpy(), w_fmt, "int8dyn", W, tag=f"step {t}",
                 lion=(h, t, m, v) if opt == "lion" else None)
        W, m, v = ref["W"], ref["m"], ref["v"]


@pytest.mark.parametrize("Nn,Kn", [(N, K), (N3, K3)])
def test_dynamic_map_fused_equals_unfused_bitwise(lib, Nn, Kn):
    _say("dynamic map fused vs unfused", Nn, Kn)
    rng = np.random.default_rng(73)
    h = synth.default_hyper("adamw")
    W = synth.random_weight(74, Nn, Kn, "bf16")
    m, v = _init_states("adamw", "int8dyn", rng, Nn, Kn)
    X, dY = synth.gaussian_case(385, T, Nn, Kn, "bf16")
    a = P.DeviceStep(W, m, v, "bf16", "int8dyn")
    b = P.DeviceStep(W, m, v, "bf16", "int8dyn")
    pa = a.fused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    pb, _ = b.unfused(lib, X, dY, "adamw", h, 2, 9, preround=True)
    torch.cuda.synchronize()
    assert torch.equal(pa, pb)
    for x, y in zip(a.host(), b.host()):
        if isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        else:
            assert np.array_equal(x, y)
