"""GPU parity at the largest inputs the boundary accepts: X or dY of just under 4 GiB, so the
kernels' 32-bit buffer offsets reach the top of their range.

The inputs are periodic small integers generated on the device (X[t, k] = (t + k) mod 8 - 4,
dY[t, n] = (3 t + n) mod 5 - 2, W[n, k] = (n + 2 k) mod 7 - 3), so every product and every fp32
sum is exact and the exact result has a closed form over one period of the token index (40
tokens for dW, 5 for dX): the host computes it in float64 from the period's residues and the
count of tokens in each.
  * the wgrad GEMM: the whole fp32 dW bitwise against the closed form;
  * the fused AdamW step: W, m, v bitwise against the unfused path, and against the oracle's
    rule on the exact gradient (plain bar);
  * dgrad: the whole bf16 dX bitwise against the nearest-even rounding of the closed form;
  * the one-launch backward step bitwise against the two-launch one.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import numerics, wgrad
from tests import parity as P

pytestmark = pytest.mark.gpu

# (T + 128) K 2 < 2^32 for X of the GEMM and the step; (T + 256) N 2 < 2^32 for dY of dgrad
T_W, N_W, K_W = 130943, 256, 16384
T_D, N_D, K_D = 130815, 16384, 256


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def _periodic(rows, cols, a, b, mod, off, chunk=2048):
    """bf16 [rows, cols] with element (i, j) = (a i + b j) mod `mod` - off, built on the device."""
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    j = torch.arange(cols, device="cuda")[None, :]
    for r0 in range(0, rows, chunk):
        i = torch.arange(r0, min(rows, r0 + chunk), device="cuda")[:, None]
        out[r0:r0 + i.shape[0]] = ((a * i + b * j) % mod - off).to(torch.bfloat16)
    return out


def _counts(T, period):
    r = np.arange(period)
    return (T // period + (r < T % period)).astype(np.float64)


def _dw_exact(T, N, K):
    """sum_t dY[t, n] X[t, k] for the periodic inputs, exactly (float64 integers)."""
    r = np.arange(40)[:, None]
    F = ((r + np.arange(K)[None, :]) % 8 - 4).astype(np.float64)          # X[t, k], t = r mod 40
    G = ((3 * r + np.arange(N)[None, :]) % 5 - 2).astype(np.float64)      # dY[t, n]
    return G.T @ (_counts(T, 40)[:, None] * F)


def test_wgrad_gemm_and_step_at_the_offset_limit(lib):
    _say("max size: wgrad GEMM and fused step", T_W, N_W, K_W, "X of", T_W * K_W * 2 / 2 ** 30, "GiB")
    X = _periodic(T_W, K_W, 1, 1, 8, 4)
    dY = _periodic(T_W, N_W, 3, 1, 5, 2)
    g = _dw_exact(T_W, N_W, K_W)
    assert np.abs(g).max() < 2 ** 24                                        # exact in fp32
    dW = torch.empty((N_W, K_W), dtype=torch.float32, device="cuda")
    lib.wgrad_gemm(X, dY, dW)
    got = dW.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, g), f"{int(np.sum(got != g))} elements of dW differ from the exact sums"

    h = synth.default_hyper("adamw")
    W = synth.random_weight(121, N_W, K_W, "bf16")
    m, v = wgrad.init_states("adamw", N_W, K_W, "f32")
    a = P.DeviceStep(W, m, v, "bf16", "f32")
    b = P.DeviceStep(W, m, v, "bf16", "f32")
    pre = torch.empty((N_W, K_W), dtype=torch.float32, device="cuda")
    lib.wgrad_step(X, dY, a.W, a.m, a.v, opt="adamw", hyper=h, step=1, seed=5, w_preround_out=pre)
    lib.optimizer_step(dW, b.W, b.m, b.v, opt="adamw", hyper=h, step=1, seed=5)
    for x, y, name in zip(a.host(), b.host(), ("W", "m", "v")):
        assert np.array_equal(x, y), f"fused and unfused {name} differ"
    ref = wgrad.step(None, None, W, m, v, "adamw", h, 1, 5, "bf16", "f32", g=g)
    gW, gm, gv = a.host()
    P.compare(ref, gW, gm, gv, pre.cpu().numpy(), "bf16", "f32", W, tag="max size")


def test_dgrad_at_the_offset_limit(lib):
    _say("max size: dgrad", T_D, N_D, K_D, "dY of", T_D * N_D * 2 / 2 ** 30, "GiB")
    dY = _periodic(T_D, N_D, 3, 1, 5, 2)
    W = _periodic(N_D, K_D, 1, 2, 7, 3)
    dX = torch.empty((T_D, K_D), dtype=torch.bfloat16, device="cuda")
    lib.dgrad(dY, W, dX)
    r = np.arange(5)[:, None]
    G5 = ((3 * r + np.arange(N_D)[None, :]) % 5 - 2).astype(np.float64)    # dY[t, :] for t = r mod 5
    Wm = ((np.arange(N_D)[:, None] + 2 * np.arange(K_D)[None, :]) % 7 - 3).astype(np.float64)
    cls = G5 @ Wm
    assert np.abs(cls).max() < 2 ** 24
    want = numerics.bf16_rne(cls.astype(np.float32))[np.arange(T_D) % 5]
    got = dX.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} elements of dX differ"


def test_one_launch_backward_at_the_offset_limit(lib):
    _say("max size: one-launch backward step vs two launches", T_D, N_D, K_D)
    dY = _periodic(T_D, N_D, 3, 1, 5, 2)
    X = _periodic(T_D, K_D, 1, 1, 8, 4)
    h = synth.default_hyper("adamw")
    W0 = synth.random_weight(122, N_D, K_D, "bf16")
    m, v = wgrad.init_states("adamw", N_D, K_D, "f32")
    outs = []
    for fused in (True, False):
        d = P.DeviceStep(W0, m, v, "bf16", "f32")
        dX = torch.empty((T_D, K_D), dtype=torch.bfloat16, device="cuda")
        kw = dict(opt="adamw", hyper=h, step=1, seed=6)
        if fused:
            ws = lib.linear_backward_step_fused(X, dY, d.W, dX, d.m, d.v, **kw)
            torch.cuda.synchronize()
            assert int(ws[1].item()) == 0
        else:
            lib.linear_backward_step(X, dY, d.W, dX, d.m, d.v, **kw)
        outs.append((dX.view(torch.int16).cpu().numpy(),) + d.host())
        del dX
    for a, b, name in zip(outs[0], outs[1], ("dX", "W", "m", "v")):
        assert np.array_equal(a, b), name
