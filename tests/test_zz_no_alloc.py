"""The allocation-free entry point (forge_linear_backward_step_fused_noalloc) against the
workspace entry point it is a variant of (forge_linear_backward_step_fused), through the C ABI:
bitwise dX, W, m, v on two calls in a row, the second on a smaller layer, so the library's one
counter array is reused and must be cleared in between.
"""
import numpy as np
import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def _pair(lib, opt, state_fmt, Tn, Nn, Kn, seed):
    rng = np.random.default_rng(seed)
    h = synth.default_hyper(opt)
    W = synth.random_weight(seed + 1, Nn, Kn, "bf16")
    m, v = P.init_states(opt, state_fmt, rng, Nn, Kn)
    X, dY = synth.gaussian_case(seed + 2, Tn, Nn, Kn, "bf16")
    Xd, _ = P.dev_operand(X)
    Dd, _ = P.dev_operand(dY)
    a = P.DeviceStep(W, m, v, "bf16", state_fmt)
    b = P.DeviceStep(W, m, v, "bf16", state_fmt)
    dXa = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    dXb = torch.empty((Tn, Kn), dtype=torch.bfloat16, device="cuda")
    kw = dict(opt=opt, hyper=h, step=3, seed=17)
    ws = lib.linear_backward_step_fused(Xd, Dd, a.W, dXa, a.m, a.v, m_scale=a.ms, v_scale=a.vs,
                                        state_map=a.state_map, **kw)
    lib.linear_backward_step_fused_noalloc(Xd, Dd, b.W, dXb, b.m, b.v, m_scale=b.ms, v_scale=b.vs,
                                           state_map=b.state_map, **kw)
    torch.cuda.synchronize()
    assert int(ws[1].item()) == 0
    assert torch.equal(dXa.view(torch.int16), dXb.view(torch.int16)), "dX"
    for x, y, name in zip(a.host(), b.host(), ("W", "m", "v")):
        if x is None:
            continue
        if isinstance(x, tuple):
            assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1]), name
        else:
            assert np.array_equal(x, y), name


def test_no_alloc_equals_workspace_entry_point_twice(lib):
    _say("no-alloc backward step, call 1: 1000 x 2048 x 4096 AdamW fp32 moments")
    _pair(lib, "adamw", "f32", 1000, 2048, 4096, 501)
    _say("no-alloc backward step, call 2 (smaller): 300 x 512 x 1024 Lion int8 moments")
    _pair(lib, "lion", "int8", 300, 512, 1024, 511)


def test_no_alloc_rejects_k_beyond_its_counters(lib):
    """K beyond the static array's 520960 columns is refused before anything is launched."""
    _say("no-alloc K limit")
    T, N, K = 1, 256, 520960 + 128
    X = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception, match="allocation-free"):
        lib.linear_backward_step_fused_noalloc(X, dY, W, dX, None, None, opt="sgd", hyper=synth.default_hyper("sgd"),
                                               step=1, seed=1)
