"""GPU checks of properties the pages state or that any correct kernel must have.

  * shard invariance (FORGE explainer, gist.science, Technical Summary section 2
    "Distributed Training Compatibility": exact under tensor parallelism, because a shard's
    gradient is complete at backward time): the step on a column slice (row-parallel shard,
    a slice of X's columns) and on a row slice (column-parallel shard, a slice of dY's columns)
    of a layer gives bitwise the same fp32 weight before rounding and the same moments as that
    slice of the full layer's step.  The stochastic-rounding key is the element's index in the
    tensor the call sees, so the shard's bf16 weight may differ by one ULP;
  * the gradient stays fp32 (section 2 "Precision and Fidelity", section 3): the device's
    moments match the oracle with the fp32 gradient and visibly differ from an oracle that
    first rounds the gradient to bf16 (negative control);
  * no write outside the outputs: every output lies between two guard bands of a known byte
    pattern that must be intact after the call, on every tile path;
  * NaN and infinity propagate: a NaN input element makes its whole gradient column NaN and an
    infinite one its row non-finite; the device's non-finite outputs are exactly the oracle's
    and all other elements meet the exact-input bar.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import numerics, wgrad
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    if not os.path.exists(forge.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def _slice_op(op: synth.Operand, c0, c1) -> synth.Operand:
    return synth.Operand(op.fmt, np.ascontiguousarray(op.data[:, c0:c1]), op.scale)


def _slice_state(st, r0, r1, c0, c1):
    if st is None:
        return None
    if isinstance(st, tuple):
        return (np.ascontiguousarray(st[0][r0:r1, c0:c1]), np.ascontiguousarray(st[1][r0:r1, c0 // 64:c1 // 64]))
    return np.ascontiguousarray(st[r0:r1, c0:c1])


def _same_state(a, b, what):
    if a is None:
        assert b is None
        return
    if isinstance(a, tuple):
        assert np.array_equal(a[0], b[0]), f"{what} codes"
        assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32)), f"{what} scales"
    else:
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


# full layer -> (column shard, row shard): [4096, 4224] at T = 200 runs 512 256 x 128 tiles and
# 32 half tiles (bf16) or 528 256 x 128 tiles (fp8); the shards run half tiles.  [4096, 4096] at
# T = 8192 runs 256 x 256 tiles; its shards the 256 x 128 path.
SHARD = [("adamw", "bf16", "f32", 4096, 4224, 200), ("lion", "bf16", "int8", 4096, 4224, 200),
         ("adamw", "fp8", "f32", 4096, 4224, 200), ("nadam", "bf16", "f32", 4096, 4096, 8192)]


@pytest.mark.parametrize("opt,in_fmt,state_fmt,N,K,T", SHARD, ids=["-".join(map(str, c)) for c in SHARD])
def test_shard_invariance(lib, opt, in_fmt, state_fmt, N, K, T):
    rng = np.random.default_rng(61)
    h = synth.default_hyper(opt)
    X, dY = synth.gaussian_case(610, T, N, K, in_fmt)
    W = synth.random_weight(62, N, K, "bf16")
    m, v = P.init_states(opt, state_fmt, rng, N, K)
    _say("shard invariance full", opt, in_fmt, state_fmt, N, K, T)
    full = P.DeviceStep(W, m, v, "bf16", state_fmt)
    pre = full.fused(lib, X, dY, opt, h, 3, 17, preround=True).cpu().numpy()
    fW, fm, fv = full.host()
    del full
    shards = {"columns 1024:3072 (row-parallel)": (0, N, 1024, 3072), "rows 1024:3072 (column-parallel)": (1024, 3072, 0, K)}
    for name, (r0, r1, c0, c1) in shards.items():
        _say("shard invariance", name)
        Xs = _slice_op(X, c0, c1)
        dYs = _slice_op(dY, r0, r1)
        s = P.DeviceStep(np.ascontiguousarray(W[r0:r1, c0:c1]), _slice_state(m, r0, r1, c0, c1),
                         _slice_state(v, r0, r1, c0, c1), "bf16", state_fmt)
        spre = s.fused(lib, Xs, dYs, opt, h, 3, 17, preround=True).cpu().numpy()
        sW, sm, sv = s.host()
        del s
        assert np.array_equal(spre.view(np.uint32), np.ascontiguousarray(pre[r0:r1, c0:c1]).view(np.uint32)), \
            f"{name}: weight before rounding differs"
        _same_state(sm, _slice_state(fm, r0, r1, c0, c1), f"{name} m")
        _same_state(sv, _slice_state(fv, r0, r1, c0, c1), f"{name} v")
        assert int(P.ulp_distance(sW, fW[r0:r1, c0:c1]).max()) <= 1, f"{name}: bf16 weight more than 1 ULP apart"


def test_gradient_is_not_rounded_to_bf16(lib):
    """Negative control: the device's step matches the oracle with the fp32 gradient and would
    fail the same bar against an oracle that rounds the gradient to bf16 first."""
    _say("fp32 gradient negative control")
    N, K, T = 2048, 4096, 200
    h = synth.default_hyper("adamw")
    X, dY = synth.gaussian_case(630, T, N, K, "bf16")
    W = synth.random_weight(631, N, K, "bf16")
    m, v = wgrad.init_states("adamw", N, K, "f32")
    g = wgrad.wgrad(wgrad.decode_operand(X), wgrad.decode_operand(dY))
    ref = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 5, "bf16", "f32", g=g)
    g16 = numerics.bf16_to_f64(numerics.bf16_rne(g.astype(np.float32)))
    ref16 = wgrad.step(X, dY, W, m, v, "adamw", h, 1, 5, "bf16", "f32", g=g16)
    d = P.DeviceStep(W, m, v, "bf16", "f32")
    d.fused(lib, X, dY, "adamw", h, 1, 5)
    _, gm, gv = d.host()
    lo, hi, mom = P.envelope("adamw", h, 1, g, P.grad_bound(X, dY), W, m, v, "bf16", "f32")
    P.moment_close(gm, ref["m64"], "m (fp32 gradient)", *mom["m"])
    P.norm_gate(gm, ref["m64"], "m (fp32 gradient)")
    rel = np.abs(gm.astype(np.float64) - ref16["m64"]) / np.maximum(np.abs(ref16["m64"]), 1e-30)
    frac = float(np.mean(rel > 1e-4))
    print(f"  against a bf16-rounded gradient: {frac:.1%} of m beyond rel 1e-4, norm ratio "
          f"{float(np.linalg.norm(gm - ref16['m64']) / np.linalg.norm(ref16['m64'])):.2e}", flush=True)
    assert frac > 0.5
    with pytest.raises(AssertionError):
        P.norm_gate(gm, ref16["m64"], "m (bf16 gradient)")


# ----------------------------------------------------------------------------- guard bands
GUARD = 1 << 20          # bytes before and after every output
PATTERN = 0xA5


class Guarded:
    """A [rows, cols] tensor of `dtype` placed between two guard bands of PATTERN bytes."""

    def __init__(self, rows, cols, dtype, init=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = rows * cols * esz
        self.buf = torch.full((2 * GUARD + n,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(rows, cols)
        if init is not None:
            self.t.copy_(init)
        assert self.t.data_ptr() % 256 == 0

    def intact(self) -> bool:
        torch.cuda.synchronize()
        return bool(torch.all(self.buf[:GUARD] == PATTERN)) and bool(torch.all(self.buf[-GUARD:] == PATTERN))


class GuardedScale(Guarded):
    def __init__(self, n):
        super().__init__(1, n, torch.float32)
        self.t = self.t.view(-1)
        self.t.zero_()


CANARY = [("bf16", "f32", 4096, 4224, 200), ("bf16", "int8", 4096, 4224, 200), ("bf16", "f32", 4096, 4096, 8192),
          ("fp8", "f32", 4096, 4224, 200), ("fp8", "int8", 4096, 4096, 8192), ("f32", "f32", 256, 384, 200),
          ("bf16", "int8", 256, 384, 200)]


@pytest.mark.parametrize("in_fmt,state_fmt,N,K,T", CANARY, ids=["-".join(map(str, c)) for c in CANARY])
def test_outputs_stay_inside_their_buffers(lib, in_fmt, state_fmt, N, K, T):
    _say("guard bands", in_fmt, state_fmt, N, K, T)
    w_dt = torch.float32 if in_fmt == "f32" else torch.bfloat16
    X, dY = synth.gaussian_case(640, T, N, K, in_fmt)
    Xd, xs = P.dev_operand(X)
    Dd, ds = P.dev_operand(dY)
    W = Guarded(N, K, w_dt, torch.randn((N, K), device="cuda").to(w_dt) * 0.02)
    pre = Guarded(N, K, torch.float32)
    if state_fmt == "f32":
        m, v = Guarded(N, K, torch.float32, torch.zeros(())), Guarded(N, K, torch.float32, torch.zeros(()))
        ms = vs = None
    else:
        m, v = Guarded(N, K, torch.int8, torch.zeros(())), Guarded(N, K, torch.uint8, torch.zeros(()))
        ms, vs = GuardedScale(N * K // 64), GuardedScale(N * K // 64)
    outs = [W, pre, m, v] + ([ms, vs] if ms is not None else [])
    h = synth.default_hyper("adamw")
    for t in (1, 2):
        lib.wgrad_step(Xd, Dd, W.t, m.t, v.t, opt="adamw", hyper=h, step=t, seed=3, x_scale=xs, dy_scale=ds,
                       m_scale=None if ms is None else ms.t, v_scale=None if vs is None else vs.t, w_preround_out=pre.t)
    assert all(o.intact() for o in outs), "the fused step wrote outside an output buffer"
    # the unfused path: the gradient buffer and the optimizer kernel's outputs
    dW = Guarded(N, K, torch.float32)
    lib.wgrad_gemm(Xd, Dd, dW.t, x_scale=xs, dy_scale=ds)
    lib.optimizer_step(dW.t, W.t, m.t, v.t, opt="adamw", hyper=h, step=3, seed=3,
                       m_scale=None if ms is None else ms.t, v_scale=None if vs is None else vs.t, w_preround_out=pre.t)
    assert all(o.intact() for o in outs + [dW]), "the unfused path wrote outside an output buffer"
    if in_fmt == "bf16":
        dX = Guarded(T, K, torch.bfloat16)
        lib.dgrad(Dd, W.t, dX.t)
        assert dX.intact(), "dgrad wrote outside dX"


# ----------------------------------------------------------------------------- NaN and infinity
NONFINITE = [("adamw", "bf16", "f32", 4096, 4224), ("sgd", "bf16", "f32", 4096, 4224), ("adamw", "bf16", "int8", 4096, 4224),
             ("adamw", "fp8", "f32", 4096, 4224), ("rmsprop", "f32", "f32", 256, 384)]


@pytest.mark.parametrize("opt,in_fmt,state_fmt,N,K", NONFINITE, ids=["-".join(map(str, c)) for c in NONFINITE])
def test_nan_and_infinity_propagate(lib, opt, in_fmt, state_fmt, N, K):
    _say("non-finite inputs", opt, in_fmt, state_fmt, N, K)
    T = 200
    h = synth.default_hyper(opt)
    w_fmt = "f32" if in_fmt == "f32" else "bf16"
    X, dY = synth.integer_case(650, T, N, K, in_fmt)
    # a NaN in X[5, 100] (gradient column 100) and an infinity in dY[7, r] (gradient row r)
    r = N - 5
    Xd_, dYd_ = X.data.copy(), dY.data.copy()
    if in_fmt == "f32":
        Xd_[5, 100], dYd_[7, r] = np.nan, np.inf
    elif in_fmt == "bf16":
        Xd_[5, 100], dYd_[7, r] = 0x7FC0, 0x7F80
    else:
        Xd_[5, 100], dYd_[7, r] = 0x7F, 0x7F            # e4m3 has no infinity: two NaNs
    X, dY = synth.Operand(X.fmt, Xd_, X.scale), synth.Operand(dY.fmt, dYd_, dY.scale)
    W = synth.random_weight(651, N, K, w_fmt)
    m, v = wgrad.init_states(opt, N, K, state_fmt)
    ref = wgrad.step(X, dY, W, m, v, opt, h, 1, 9, w_fmt, state_fmt)
    d = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    pre = d.fused(lib, X, dY, opt, h, 1, 9, preround=True).cpu().numpy().astype(np.float64)
    gW, gm, gv = d.host()
    gW64 = numerics.bf16_to_f64(gW) if w_fmt == "bf16" else gW.astype(np.float64)
    rW64 = numerics.bf16_to_f64(ref["W"]) if w_fmt == "bf16" else ref["W"].astype(np.float64)
    fin = np.isfinite(ref["W64"])
    assert (~fin).sum() >= N + K - 1, "the planted values must reach a whole row and column"
    for what, a, b in (("W before rounding", pre, ref["W64"]), ("W", gW64, rW64)):
        assert np.array_equal(np.isnan(a), np.isnan(b)), f"{what}: NaN positions differ"
        assert np.array_equal(np.isposinf(a), np.isposinf(b)) and np.array_equal(np.isneginf(a), np.isneginf(b)), \
            f"{what}: infinite positions differ"
    for name, got in (("m", gm), ("v", gv)):
        if got is None:
            continue
        if state_fmt == "f32":
            a, b = got.astype(np.float64), ref[f"{name}64"]
            assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(np.isinf(a), np.isinf(b)), name
        else:
            sc, rs = got[1], ref[name][1]
            assert np.array_equal(np.isnan(sc), np.isnan(rs)), f"{name}: NaN block scales differ"
            assert np.all(got[0][np.repeat(np.isnan(sc), 64, axis=1)] == 0), f"{name}: codes of non-finite blocks"
    # every finite element meets the exact-input bar (its gradient is an exact sum)
    keep_rows = np.flatnonzero(np.arange(N) != r)
    assert np.all(fin[keep_rows][:, np.arange(K) != 100])
    c0 = 128
    cols = np.arange(c0, c0 + 64)
    assert np.all(fin[np.ix_(keep_rows, cols)])
    sub = lambda a: None if a is None else (
        (a[0][np.ix_(keep_rows, cols)], a[1][keep_rows][:, c0 // 64:c0 // 64 + 1]) if isinstance(a, tuple)
        else a[np.ix_(keep_rows, cols)])
    ref_s = {k: (sub(val) if isinstance(val, (np.ndarray, tuple)) else val) for k, val in ref.items()}
    P.compare(ref_s, sub(gW), sub(gm), sub(gv), pre[np.ix_(keep_rows, cols)], w_fmt, state_fmt, sub(W),
              tag="finite elements")
