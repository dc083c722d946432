"""The C ABI on the host, no GPU needed: the library loads, exports every symbol include/forge.h
declares, rejects bad arguments with the documented status before touching any buffer, and
hands the kernels the per-step scalars the oracle's rules use.

The bad-argument calls pass fake, never-dereferenced addresses: validation happens before
any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import optimizers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def forge():
    import optimizer_step_weight_amd as f
    if not os.path.exists(f.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    f._lib()
    return f


def test_exports_every_declared_symbol(forge):
    inc = os.path.join(ROOT, "include")
    hdr = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    names = sorted(set(re.findall(r"\b(forge_[a-z_0-9]+)\s*\(", hdr)))
    assert len(names) >= 13 and "forge_clock_sample" in names
    L = forge._lib()
    for n in names:
        assert hasattr(L, n), n
    assert forge.version() == 100
    assert forge.status_string(0) == "ok" and forge.status_string(5) == "overlapping buffers"


def test_build_id_matches_the_sources(forge):
    """The library embeds the hash of the sources it was built from; the binding refuses a stale one."""
    from optimizer_step_weight_amd import _build
    assert forge.build_id() == _build.source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", forge.build_id())


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _t(f, rows, cols, dtype, off=0, scale=None, ld=None):
    return f.Tensor(FAKE + off, dtype, rows, cols, cols if ld is None else ld, scale)


def _call_step(f, X, dY, W, m, v, opt=0, step=1, hyper=None, opts=None):
    h = f._hyper(hyper or synth.default_hyper("adamw"))
    r = ctypes.byref
    return f._lib().forge_wgrad_step(r(X) if X else None, r(dY) if dY else None, r(W) if W else None,
                                     r(m) if m else None, r(v) if v else None, r(h), opt, step, 1,
                                     r(opts) if opts else None, None)


def test_validation_codes(forge):
    f = forge
    GB = 1 << 30
    T, N, K = 64, 256, 384
    X = lambda **k: _t(f, T, K, f.BF16, 0 * GB, **k)
    dY = lambda **k: _t(f, T, N, f.BF16, 1 * GB, **k)
    W = lambda dt=f.BF16, r=N, c=K, off=2 * GB: _t(f, r, c, dt, off)
    m = lambda dt=f.F32, off=3 * GB: _t(f, N, K, dt, off)
    v = lambda dt=f.F32, off=4 * GB: _t(f, N, K, dt, off)
    ok = (X(), dY(), W(), m(), v())
    cases = [
        ((None, dY(), W(), m(), v()), {}, 1),                                # null X
        (ok, dict(step=0), 1),                                               # step < 1
        (ok, dict(opt=9), 1),                                                # unknown rule
        ((X(), dY(), W(), None, v()), {}, 1),                                # AdamW needs m
        ((X(), dY(), W(), m(), v()), dict(opt=6), 1),                        # SGD keeps no state
        ((X(), dY(), W(r=128), m(), v()), {}, 2),                            # W rows != N
        ((_t(f, T, 200, f.BF16), dY(), W(c=200), m(), v()), {}, 2),          # K % 128
        ((X(), _t(f, T + 1, N, f.BF16, GB), W(), m(), v()), {}, 2),          # token counts differ
        ((_t(f, T, K, f.F32), dY(), W(), m(), v()), {}, 3),                  # mixed input dtypes
        ((X(), dY(), W(dt=f.I8_B64), m(), v()), {}, 3),                      # bad weight dtype
        ((X(), dY(), W(), m(dt=f.U8_B64), v()), {}, 3),                      # m must be signed
        ((X(), dY(), W(), _t(f, N, K, f.I8_B64, 3 * GB, scale=FAKE + 5 * GB), v()), {}, 3),  # m int8, v fp32
        ((_t(f, T, K, f.BF16, 8), dY(), W(), m(), v()), {}, 4),              # misaligned
        ((_t(f, T, K, f.BF16, ld=2 * K), dY(), W(), m(), v()), {}, 4),       # X rows not contiguous
        ((X(), dY(), W(), m(), _t(f, N, K, f.F32, 4 * GB, ld=K + 4)), {}, 4),  # v rows not contiguous
        ((X(), dY(), W(off=0), m(), v()), {}, 5),                            # W aliases X
        ((X(), dY(), W(), m(off=2 * GB + 4096 * 16), v()), {}, 5),         # m overlaps W
        ((_t(f, T, K, f.FP8_E4M3), _t(f, T, N, f.FP8_E4M3, GB), W(), m(), v()), {}, 1),  # fp8 without scales
    ]
    for args, kw, want in cases:
        got = _call_step(f, *args, **kw)
        assert got == want, (got, want, f.last_error())
        assert f.last_error()
    # int8 states need their block scales
    assert _call_step(f, X(), dY(), W(), m(dt=f.I8_B64), v(dt=f.U8_B64)) == 1
    # an empty weight is a valid no-op that touches nothing (N = 0)
    assert _call_step(f, X(), _t(f, T, 0, f.BF16, GB), W(r=0), m(), _t(f, 0, K, f.F32, 4 * GB)) in (0, 2)


def test_dgrad_and_unfused_validation(forge):
    f = forge
    GB = 1 << 30
    r = ctypes.byref
    L = f._lib()
    dY, W, dX = _t(f, 100, 256, f.BF16), _t(f, 256, 384, f.BF16, GB), _t(f, 100, 384, f.BF16, 2 * GB)
    assert L.forge_dgrad(r(dY), r(W), r(_t(f, 100, 256, f.BF16, 2 * GB)), None) == 2
    assert L.forge_dgrad(r(dY), r(W), r(_t(f, 100, 384, f.F32, 2 * GB)), None) == 3
    assert L.forge_dgrad(r(dY), r(W), r(_t(f, 100, 384, f.BF16, 0)), None) == 5
    assert L.forge_dgrad(r(dY), r(_t(f, 256, 384, f.BF16, GB, ld=512)), r(dX), None) == 4
    # 32-bit offsets: W of 2^31 elements, or dY that reaches 2^31 elements with one tile of tokens
    assert L.forge_dgrad(r(_t(f, 100, 131072, f.BF16)), r(_t(f, 131072, 16384, f.BF16, GB)),
                         r(_t(f, 100, 16384, f.BF16, 2 * GB)), None) == 2
    assert L.forge_dgrad(r(_t(f, 131072 - 256, 16384, f.BF16)), r(_t(f, 16384, 128, f.BF16, 8 * GB)),
                         r(_t(f, 131072 - 256, 128, f.BF16, 9 * GB)), None) == 2
    X = _t(f, 100, 384, f.BF16, 3 * GB)
    assert L.forge_wgrad_gemm(r(X), r(dY), r(_t(f, 256, 384, f.BF16, 4 * GB)), None) == 3
    assert L.forge_wgrad_gemm(r(X), r(dY), r(_t(f, 256, 256, f.F32, 4 * GB)), None) == 2
    h = f._hyper(synth.default_hyper("sgd"))
    dW = _t(f, 256, 384, f.F32, 4 * GB)
    assert L.forge_optimizer_step(r(dW), r(_t(f, 256, 384, f.BF16, 4 * GB)), None, None, r(h), 6, 1, 0, None, None) == 5


def test_one_launch_backward_validation(forge):
    """forge_linear_backward_step_fused: the backward step's checks, its own shape rule
    (N % 256, K % 128) and the workspace's size, alignment and aliasing."""
    f = forge
    GB = 1 << 30
    r = ctypes.byref
    L = f._lib()
    T, N, K = 100, 256, 384
    assert f.backward_workspace_bytes(K) == 4 * (26 + K // 128)
    assert f.backward_workspace_bytes(-1) == -1
    h = f._hyper(synth.default_hyper("adamw"))
    need = f.backward_workspace_bytes(K)

    def call(X=None, dY=None, W=None, dX=None, m=None, v=None, ws=FAKE + 9 * GB, nbytes=need):
        X = X or _t(f, T, K, f.BF16)
        dY = dY or _t(f, T, N, f.BF16, GB)
        W = W or _t(f, N, K, f.BF16, 2 * GB)
        dX = dX or _t(f, T, K, f.BF16, 3 * GB)
        m = m or _t(f, W.rows, W.cols, f.F32, 4 * GB)
        v = v or _t(f, W.rows, W.cols, f.F32, 5 * GB)
        return L.forge_linear_backward_step_fused(r(X), r(dY), r(W), r(dX), r(m), r(v), r(h), 0, 1, 1, None, ws,
                                                  nbytes, None)

    assert call(ws=None) == 1                                             # no workspace
    assert call(nbytes=need - 4) == 1                                     # workspace too small
    assert call(ws=FAKE + 9 * GB + 2) == 4                                # workspace misaligned
    assert call(ws=FAKE + 2 * GB + 64) == 5                               # workspace inside W
    assert call(ws=FAKE + 3 * GB) == 5                                    # workspace is dX
    assert call(dX=_t(f, T, K, f.F32, 3 * GB)) == 3                       # dX must be bf16
    assert call(dX=_t(f, T, K, f.BF16, 2 * GB)) == 5                      # dX overlaps W
    dY128 = _t(f, T, 128, f.BF16, GB)                                     # N = 128: not a multiple of 256
    assert call(dY=dY128, W=_t(f, 128, K, f.BF16, 2 * GB)) == 2
    assert "256" in f.last_error()
    # the same arguments are accepted by the two-launch entry point's checks up to the device
    X, dY, W, dX = _t(f, T, K, f.BF16), dY128, _t(f, 128, K, f.BF16, 2 * GB), _t(f, T, K, f.BF16, 3 * GB)
    m, v = _t(f, 128, K, f.F32, 4 * GB), _t(f, 128, K, f.F32, 5 * GB)
    assert L.forge_linear_backward_step(r(X), r(dY), r(W), r(dX), r(m), r(_t(f, 128, 200, f.F32, 5 * GB)), r(h), 0,
                                        1, 1, None, None) == 2


def test_no_alloc_backward_validation(forge):
    """The allocation-free variant: the one-launch checks, and K within its static counters
    ((4096 - 26) x 128 columns)."""
    f = forge
    GB = 1 << 30
    r = ctypes.byref
    L = f._lib()
    h = f._hyper(synth.default_hyper("sgd"))
    T, N = 1, 256
    Kmax = (4096 - 26) * 128

    def call(K, n=N):
        return L.forge_linear_backward_step_fused_noalloc(
            r(_t(f, T, K, f.BF16)), r(_t(f, T, n, f.BF16, GB)), r(_t(f, n, K, f.BF16, 2 * GB)),
            r(_t(f, T, K, f.BF16, 3 * GB)), None, None, r(h), 6, 1, 1, None, None)

    assert call(Kmax + 128) == 2 and "allocation-free" in f.last_error()
    assert call(1024, n=128) == 2                                         # N % 256


@pytest.mark.parametrize("opt", synth.OPTIMIZERS)
@pytest.mark.parametrize("t", [1, 2, 5, 6, 50])
def test_host_scalars_match_oracle(forge, opt, t):
    h = synth.default_hyper(opt)
    s = forge.step_scalars(opt, h, t)
    ref = optimizers.step_scalars(opt, h, t)
    p = optimizers.hyper64(h)
    f32 = lambda x: float(np.float32(x))
    dec = optimizers.decoupled(opt, p["wd_mode"])
    assert s["decay"] == f32(1 - p["lr"] * p["wd"] if dec else 1.0)
    assert s["l2"] == f32(0.0 if dec else p["wd"])
    if opt == "adamw":
        assert s["c1"] == f32(p["lr"] / ref["bc1"]) and s["c2"] == f32(1 / ref["bc2"])
    if opt == "nadam":
        assert s["c1"] == pytest.approx(f32(p["lr"] * (1 - ref["mu"]) / (1 - ref["prod"])), rel=1e-6)
        assert s["c3"] == pytest.approx(f32(p["lr"] * ref["mu_next"] / (1 - ref["prod_next"])), rel=1e-6)
    if opt == "radam":
        assert s["rectified"] == float(ref["rectified"])
        want = p["lr"] * ref["r"] * np.sqrt(ref["bc2"]) / ref["bc1"] if ref["rectified"] else p["lr"] / ref["bc1"]
        assert s["c1"] == pytest.approx(f32(want), rel=1e-6)
    if opt == "rmsprop":
        assert s["b2"] == f32(p["alpha"]) and s["omb2"] == f32(1 - p["alpha"])
    if opt == "sgd_momentum":
        assert s["c1"] == f32(p["momentum"])


def test_binding_rejects_host_tensors_and_short_scales(forge):
    """The binding refuses what the C ABI cannot see: host memory and scale buffers of the wrong size."""
    import torch
    h = synth.default_hyper("adamw")
    X = torch.zeros((64, 256), dtype=torch.bfloat16)
    dY = torch.zeros((64, 256), dtype=torch.bfloat16)
    W = torch.zeros((256, 256), dtype=torch.bfloat16)
    m, v = torch.zeros((256, 256)), torch.zeros((256, 256))
    with pytest.raises(ValueError, match="CUDA tensor"):
        forge.wgrad_step(X, dY, W, m, v, opt="adamw", hyper=h, step=1, seed=1)
    m8, v8 = torch.zeros((256, 256), dtype=torch.int8), torch.zeros((256, 256), dtype=torch.uint8)
    short = torch.zeros(256 * 256 // 64 - 1)
    # each tensor's scale is checked before its device (so the checks are visible without a GPU)
    with pytest.raises(ValueError, match="1023"):
        forge._tensor(m8, short)
    with pytest.raises(ValueError, match="float32"):
        forge._tensor(v8, torch.zeros(1024, dtype=torch.float16))
    with pytest.raises(ValueError, match="takes no scale"):
        forge._tensor(m, torch.zeros(1024))
    with pytest.raises(ValueError, match="1 elements"):
        forge._tensor(torch.zeros((64, 256), dtype=torch.float8_e4m3fn), torch.zeros(2))
    with pytest.raises(ValueError, match="unit column stride"):
        forge.dgrad(dY.t(), W, torch.zeros((256, 256), dtype=torch.bfloat16))
