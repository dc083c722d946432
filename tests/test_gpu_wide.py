"""GPU tests of the wide-tile path of the fused step: 256 x 256 tiles, one 8-wave workgroup per CU.

bf16 inputs with T >= 8192 take wide tiles where K is a multiple of 256: whole rounds of wide
tiles, and where the R wide tiles leave a remainder r over the CUs, the last r / (N / 256)
256-column blocks (or the last r / (K / 256) row blocks) as 2 r half-wide tiles of 128 x 256
in the same launch, half of them dispatched first.  Otherwise whole rounds of wide tiles cover
part of the weight and the rest runs on the 256 x 128 path in a second launch.  Every
element's token sum runs in the same order on all these tiles, so the fused step must equal
the unfused path (the 256 x 128 GEMM to HBM, then the optimizer kernel) bitwise, whatever mix
of tiles and launches covers the weight.  Shapes (on 256 CUs): 4096 x 4096 is 256 wide tiles;
2048 x 8192 is 8 x 32 wide tiles; 4096 x 4224 (K / 256 not whole) takes 256 wide tiles and
runs its last 128-column block as 32 half tiles in the second launch; 6144 x 4096 is 384 wide
tiles, so its last 8 row blocks run as 256 half-wide tiles; 4096 x 5120 (320 tiles) and
2048 x 9216 (288) run their last 4 256-column blocks as 128 and 64 half-wide tiles.  T = 8193
and 8200 leave a ragged last slab of tokens.  The half-wide plan starts at T = 4096, so
4096 x 5120 and 2048 x 9216 also run at T = 4096 and 4100.  fp8 inputs have no half-wide
tiles: whole rounds of wide tiles, the rest on the 256 x 128 path.  The full-size workload tests (the
Llama-3.1-8B block at T = 8192, the optimizer sweep at T = 16384 in bf16 and fp8) check this
path against the fp64 oracle on sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests import parity as P
from tests.test_gpu_parity import _init_states, _say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    forge.device_check(0)
    return forge


def _same(a: P.DeviceStep, b: P.DeviceStep):
    for x, y in zip(a.host(), b.host()):
        if isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
        elif x is None:
            assert y is None
        else:
            assert np.array_equal(x, y)


CASES = [((4096, 4096), "adamw", "bf16", "f32", 8192), ((4096, 4224), "adamw", "bf16", "f32", 8200),
         ((2048, 8192), "lion", "bf16", "int8", 8193), ((4096, 4096), "nadam", "f32", "f32", 8192),
         ((4096, 4224), "radam", "bf16", "int8", 8192), ((2048, 8192), "rmsprop", "bf16", "f32", 8192),
         ((4096, 4096), "adagrad", "bf16", "f32", 8193), ((4096, 4224), "sgd", "f32", "f32", 8192),
         ((2048, 8192), "sgd_momentum", "bf16", "int8", 8192), ((6144, 4096), "adamw", "bf16", "f32", 8192),
         ((6144, 4096), "lion", "bf16", "int8", 8200), ((6144, 4096), "adamw", "bf16", "int8dyn", 8192),
         ((4096, 5120), "nadam", "bf16", "int8", 8193), ((2048, 9216), "adamw", "bf16", "f32", 8192),
         ((4096, 5120), "adamw", "bf16", "int8", 4096), ((2048, 9216), "lion", "f32", "f32", 4100)]


@pytest.mark.parametrize("shape,opt,w_fmt,state_fmt,Tn", CASES,
                         ids=[f"{s[0]}x{s[1]}-{o}-{w}-{st}-T{t}" for s, o, w, st, t in CASES])
def test_wide_fused_equals_unfused_bitwise(lib, shape, opt, w_fmt, state_fmt, Tn):
    Nn, Kn = shape
    _say("wide fused vs unfused", Nn, Kn, opt, w_fmt, state_fmt, "T", Tn)
    rng = np.random.default_rng(71)
    h = synth.default_hyper(opt)
    W = synth.random_weight(72, Nn, Kn, w_fmt)
    m, v = _init_states(opt, state_fmt, rng, Nn, Kn)
    a = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    b = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    for t in (1, 2):
        X, dY = synth.gaussian_case(700 + t, Tn, Nn, Kn, "bf16")
        pa = a.fused(lib, X, dY, opt, h, t, 23, preround=True)
        pb, _ = b.unfused(lib, X, dY, opt, h, t, 23, preround=True)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb), f"pre-rounding weights differ at step {t}"
        _same(a, b)


# fp8 e4m3 inputs (per-tensor scales) take the same wide tiles for T >= 8192; the rest of the
# columns run on the 256 x 128 fp8 kernel.
CASES8 = [((4096, 4096), "adamw", "bf16", "f32", 8192), ((4096, 4224), "nadam", "bf16", "int8", 8200),
          ((4096, 4096), "lion", "f32", "f32", 8193), ((2048, 8192), "sgd", "bf16", "f32", 8192),
          ((6144, 4096), "radam", "bf16", "f32", 8192)]


@pytest.mark.parametrize("shape,opt,w_fmt,state_fmt,Tn", CASES8,
                         ids=[f"fp8-{s[0]}x{s[1]}-{o}-{w}-{st}-T{t}" for s, o, w, st, t in CASES8])
def test_wide_fp8_fused_equals_unfused_bitwise(lib, shape, opt, w_fmt, state_fmt, Tn):
    Nn, Kn = shape
    _say("wide fp8 fused vs unfused", Nn, Kn, opt, w_fmt, state_fmt, "T", Tn)
    rng = np.random.default_rng(75)
    h = synth.default_hyper(opt)
    W = synth.random_weight(76, Nn, Kn, w_fmt)
    m, v = _init_states(opt, state_fmt, rng, Nn, Kn)
    a = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    b = P.DeviceStep(W, m, v, w_fmt, state_fmt)
    for t in (1, 2):
        X, dY = synth.gaussian_case(750 + t, Tn, Nn, Kn, "fp8")
        pa = a.fused(lib, X, dY, opt, h, t, 29, preround=True)
        pb, _ = b.unfused(lib, X, dY, opt, h, t, 29, preround=True)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb), f"pre-rounding weights differ at step {t}"
        _same(a, b)


def test_wide_llama_down_proj_equals_unfused(lib):
    """Llama-3.1-8B down_proj at T = 8192: 768 wide tiles and 256 half-wide tiles, one launch."""
    Nn, Kn, Tn = 4096, 14336, 8192
    _say("wide fused vs unfused, down_proj T=8192")
    g = torch.Generator(device="cuda").manual_seed(11)
    X = torch.randn((Tn, Kn), device="cuda", generator=g).to(torch.bfloat16)
    dY = (torch.randn((Tn, Nn), device="cuda", generator=g) * 1e-3).to(torch.bfloat16)
    W0 = (torch.randn((Nn, Kn), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    h = synth.default_hyper("adamw")
    Wa, Wb = W0.clone(), W0.clone()
    ma, va = torch.zeros((Nn, Kn), device="cuda"), torch.zeros((Nn, Kn), device="cuda")
    mb, vb = torch.zeros_like(ma), torch.zeros_like(va)
    dW = torch.empty((Nn, Kn), device="cuda")
    for t in (1, 2):
        lib.wgrad_step(X, dY, Wa, ma, va, opt="adamw", hyper=h, step=t, seed=99)
        lib.wgrad_gemm(X, dY, dW)
        lib.optimizer_step(dW, Wb, mb, vb, opt="adamw", hyper=h, step=t, seed=99)
    torch.cuda.synchronize()
    assert torch.equal(Wa, Wb) and torch.equal(ma, mb) and torch.equal(va, vb)
