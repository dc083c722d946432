"""GPU parity of the one-launch backward step (forge_linear_backward_step_fused): dX from the
weight before the step and the fused step, in one grid of dX tiles and step tiles taken from
per-XCD-slot work queues.

  * against the oracle: exact-sum X and dY (the gradient is exact, so W, m, v meet the plain
    bar), dX within one bf16 ULP plus the fp32 summation bound of its N products;
  * against the two-launch path (forge_linear_backward_step): bitwise dX, W, m, v on Gaussian
    inputs where both use the same tile shapes, and at the workloads' long token counts;
  * a workspace holding garbage before the call, token counts that are not whole tiles, and the
    error word left at 0.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import numerics, optimizers, wgrad
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(lib, fused, X, dY, d, dX, opt, h, step, seed, pre=None, workspace=None):
    Xd, _ = P.dev_operand(X)
    Dd, _ = P.dev_operand(dY)
    kw = dict(opt=opt, hyper=h, step=step, seed=seed, m_scale=d.ms, v_scale=d.vs, w_preround_out=pre,
              state_map=d.state_map)
    if fused:
        return lib.linear_backward_step_fused(Xd, Dd, d.W, dX, d.m, d.v, workspace=workspace, **kw)
    lib.linear_backward_step(Xd, Dd, d.W, dX, d.m, d.v, **kw)
    return None


def _error_word(ws):
    torch.cuda.synchronize()
    return int(ws[1].item())


# (opt, state format, T, N, K): shapes with half tiles only (256 x 384, 1024 x 4096), full and
# half tiles (2048 x 4224), token counts that are not whole 256-token tiles
ORACLE = [("adamw", "f32", 200, 256, 384), ("lion", "int8", 333, 1024, 4096), ("nadam", "int8dyn", 257, 256, 384),
          ("radam", "f32", 512, 2048, 4224), ("sgd_momentum", "int8", 1, 256, 384), ("rmsprop", "f32", 255, 512, 1024)]


@pytest.mark.parametrize("opt,state_fmt,Tn,Nn,Kn", ORACLE, ids=[f"{o}-{s}-T{t}-{n}x{k}" for o, s, t, n, k in ORACLE])
def test_one_launch_matches_oracle(lib, opt, state_fmt, Tn, Nn, Kn):
    rng = np.random.default_rng(101)
    h = synth.default_hyper(opt)
    W = synth.random_weight(102, Nn, Kn, "bf16")
    m, v = P.init_states(opt, state_fmt, rng, Nn, Kn)
    for i, t in enumerate((1, 4)):
        _say("one-launch backward vs oracle", opt, state_fmt, Tn, Nn, Kn, "step", t)
        X, dY = synth.integer_case(410 + i, Tn, Nn, Kn, "bf16")
        ref = wgrad.step(X, dY, W, m, v, opt, h, t, 31, "bf16", state_fmt)
        d = P.DeviceStep(W, m, v, "bf16", state_fmt)
        dX = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
        pre = torch.empty((Nn, Kn), dtype=torch.float32, device="cuda")
        ws = _run(lib, True, X, dY, d, dX, opt, h, t, 31, pre=pre)
        assert _error_word(ws) == 0
        gW, gm, gv = d.host()
        P.compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", state_fmt, W, tag=f"step {t}",
                  lion=(h, t, m, v) if opt == "lion" else None)
        P.dx_close(_bits(dX), wgrad.decode_operand(dY), numerics.bf16_to_f64(W), "dX from the old weight")
        W, m, v = ref["W"], ref["m"], ref["v"]


# bitwise against the two-launch path: (opt, state format, T, N, K)
BITWISE = [("adamw", "f32", 200, 2048, 4224), ("lion", "int8", 1000, 1024, 4096), ("adamw", "int8dyn", 777, 4096, 1024),
           ("adagrad", "f32", 4096, 2048, 2048), ("sgd", "int8", 64, 2048, 2048)]


@pytest.mark.parametrize("opt,state_fmt,Tn,Nn,Kn", BITWISE, ids=[f"{o}-{s}-T{t}-{n}x{k}" for o, s, t, n, k in BITWISE])
def test_one_launch_equals_two_launches(lib, opt, state_fmt, Tn, Nn, Kn):
    _say("one-launch vs two launches", opt, state_fmt, Tn, Nn, Kn)
    rng = np.random.default_rng(103)
    h = synth.default_hyper(opt)
    W = synth.random_weight(104, Nn, Kn, "bf16")
    m, v = P.init_states(opt, state_fmt, rng, Nn, Kn)
    X, dY = synth.gaussian_case(420, Tn, Nn, Kn, "bf16")
    a = P.DeviceStep(W, m, v, "bf16", state_fmt)
    b = P.DeviceStep(W, m, v, "bf16", state_fmt)
    dXa = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    dXb = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    ws = torch.randint(-2 ** 31, 2 ** 31 - 1, (lib.backward_workspace_bytes(Kn) // 4,), dtype=torch.int32,
                       device="cuda")    # garbage before the call must not matter
    for t in (1, 2):
        _run(lib, True, X, dY, a, dXa, opt, h, t, 5, workspace=ws)
        _run(lib, False, X, dY, b, dXb, opt, h, t, 5)
        assert _error_word(ws) == 0
        assert torch.equal(dXa.view(torch.int16), dXb.view(torch.int16)), "dX"
        for x, y, name in zip(a.host(), b.host(), ("W", "m", "v")):
            if x is None:
                continue
            if isinstance(x, tuple):
                assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1]), name
            else:
                assert np.array_equal(x, y), name


# every rule and moment format, bitwise against the two-launch path (2048 x 2048: 128 tiles of
# 256 x 128, the smallest layer on which both paths use them)
ALL = [(o, f) for o in synth.OPTIMIZERS for f in ("f32", "int8", "int8dyn")
       if f == "f32" or optimizers.STATES[o]]


@pytest.mark.parametrize("opt,state_fmt", ALL, ids=["-".join(c) for c in ALL])
def test_one_launch_every_rule_equals_two_launches(lib, opt, state_fmt):
    _say("one-launch vs two launches, every rule", opt, state_fmt)
    Tn, Nn, Kn = 200, 2048, 2048
    rng = np.random.default_rng(107)
    h = synth.default_hyper(opt)
    W = synth.random_weight(108, Nn, Kn, "bf16")
    m, v = P.init_states(opt, state_fmt, rng, Nn, Kn)
    X, dY = synth.gaussian_case(450, Tn, Nn, Kn, "bf16")
    a = P.DeviceStep(W, m, v, "bf16", state_fmt)
    b = P.DeviceStep(W, m, v, "bf16", state_fmt)
    dXa = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    dXb = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    ws = _run(lib, True, X, dY, a, dXa, opt, h, 3, 9)
    _run(lib, False, X, dY, b, dXb, opt, h, 3, 9)
    assert _error_word(ws) == 0
    assert torch.equal(dXa.view(torch.int16), dXb.view(torch.int16)), "dX"
    for x, y, name in zip(a.host(), b.host(), ("W", "m", "v")):
        if x is None:
            continue
        if isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1]), name
        else:
            assert np.array_equal(x, y), name


@pytest.mark.parametrize("Tn", [0, 1, 255, 256, 257])
def test_one_launch_token_counts(lib, Tn):
    _say("one-launch token count", Tn)
    Nn, Kn = 512, 1024
    h = synth.default_hyper("adamw")
    W = synth.random_weight(105, Nn, Kn, "bf16")
    m, v = wgrad.init_states("adamw", Nn, Kn, "f32")
    X, dY = synth.integer_case(430, Tn, Nn, Kn, "bf16")
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 6, "bf16", "f32")
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    dX = torch.full((Tn, Kn), 7.0, dtype=torch.bfloat16, device="cuda")
    pre = torch.empty((Nn, Kn), dtype=torch.float32, device="cuda")
    ws = _run(lib, True, X, dY, d, dX, "adamw", h, 1, 6, pre=pre)
    assert _error_word(ws) == 0
    gW, gm, gv = d.host()
    P.compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, tag=f"T={Tn}")
    if Tn:
        P.dx_close(_bits(dX), wgrad.decode_operand(dY), numerics.bf16_to_f64(W), "dX")


def test_one_launch_reads_the_old_weight(lib):
    """Large steps: dX must match the weight before the update and visibly differ from the one after."""
    _say("one-launch ordering")
    Tn, Nn, Kn = 512, 1024, 2048
    X, dY = synth.gaussian_case(440, Tn, Nn, Kn, "bf16")
    W = synth.random_weight(106, Nn, Kn, "bf16")
    m, v = wgrad.init_states("adamw", Nn, Kn, "f32")
    h = synth.Hyper(lr=0.05, weight_decay=0.0)
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    dX = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    ws = _run(lib, True, X, dY, d, dX, "adamw", h, 1, 3)
    assert _error_word(ws) == 0
    got = _bits(dX)
    dY64 = wgrad.decode_operand(dY)
    P.dx_close(got, dY64, numerics.bf16_to_f64(W), "dX from the old weight")
    new_W = d.host()[0]
    with pytest.raises(AssertionError):
        P.dx_close(got, dY64, numerics.bf16_to_f64(new_W), "dX from the new weight")


# The Llama-3.1-8B layers at T = 8192 (the two-launch path takes 256 x 256 dX tiles and, for
# q/o/down, 256 x 256 step tiles there): bitwise against it.
LLAMA = [("q_proj", 4096, 4096), ("k_proj", 1024, 4096), ("down_proj", 4096, 14336)]


@pytest.mark.parametrize("name,Nn,Kn", LLAMA, ids=[x[0] for x in LLAMA])
def test_one_launch_llama_layers_equal_two_launches(lib, name, Nn, Kn):
    _say("one-launch vs two launches, Llama-3.1-8B", name, Nn, Kn, "T 8192")
    Tn = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    X = (torch.randn((Tn, Kn), generator=g, device="cuda")).to(torch.bfloat16)
    dY = (torch.randn((Tn, Nn), generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    W0 = (torch.randn((Nn, Kn), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    h = synth.default_hyper("adamw")
    outs = []
    for fused in (True, False):
        W = W0.clone()
        m = torch.zeros((Nn, Kn), dtype=torch.float32, device="cuda")
        v = torch.zeros((Nn, Kn), dtype=torch.float32, device="cuda")
        dX = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
        kw = dict(opt="adamw", hyper=h, step=1, seed=11)
        if fused:
            ws = lib.linear_backward_step_fused(X, dY, W, dX, m, v, **kw)
            assert _error_word(ws) == 0
        else:
            lib.linear_backward_step(X, dY, W, dX, m, v, **kw)
        torch.cuda.synchronize()
        outs.append((dX.view(torch.int16), W.view(torch.int16), m, v))
    for a, b, what in zip(outs[0], outs[1], ("dX", "W", "m", "v")):
        assert torch.equal(a, b), what
