"""The autograd layer (optimizer_step_weight_amd.autograd.FusedLinear) on the GPU.

* one backward against the CPU oracle: dX within the summation bound of dY W with the old
  weight (plus one bf16 ULP), W / m / v within the parity bar of the oracle's fused step on the
  same X and dY (so the wrapper passes the right tensors, in the right order, with the right
  step count);
* the weight is updated even when the layer's input needs no gradient;
* a small synthetic training loop (a two-layer ReLU network fitting a random teacher network)
  with FusedLinear layers tracks the same network trained in fp32 with torch.optim.AdamW
  (FORGE explainer, Technical Summary section 4: training with the fused step tracks fused
  AdamW within noise).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import os
    import optimizer_step_weight_amd as forge
    if not os.path.exists(forge.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    forge.device_check(0)
    return forge


def _say(*a):
    print("[case]", *a, flush=True)


def test_one_backward_matches_the_oracle(lib):
    import synth
    from oracle import numerics, wgrad
    from optimizer_step_weight_amd.autograd import FusedLinear
    from tests import parity as P
    _say("autograd one step against the oracle")
    torch.manual_seed(0)
    hyper = synth.Hyper(lr=1e-3, weight_decay=0.01)
    layer = FusedLinear(256, 512, opt="adamw", hyper=hyper, seed=7)
    W0 = P.host_weight(layer.weight, "bf16")
    x = torch.randn(200, 256, device="cuda").to(torch.bfloat16).requires_grad_(True)
    dy = (torch.randn(200, 512, device="cuda") * 1e-2).to(torch.bfloat16)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    X = synth.Operand("bf16", P.host_weight(x.detach(), "bf16"))
    dY = synth.Operand("bf16", P.host_weight(dy, "bf16"))
    # dX from the weight before the step
    P.dx_close(P.host_weight(x.grad, "bf16"), wgrad.decode_operand(dY), numerics.bf16_to_f64(W0), "dX")
    # the fused step, oracle at step 1 with the layer's seed
    m0, v0 = wgrad.init_states("adamw", 512, 256, "f32")
    ref = wgrad.step(X, dY, W0, m0, v0, "adamw", hyper, 1, 7, "bf16", "f32")
    env = P.envelope("adamw", hyper, 1, ref["g"], P.grad_bound(X, dY), W0, m0, v0, "bf16", "f32")
    P.compare(ref, P.host_weight(layer.weight, "bf16"), layer.m.cpu().numpy(), layer.v.cpu().numpy(), None,
              "bf16", "f32", W0, env, tag="autograd step 1")
    assert layer.step_count == 1 and not np.array_equal(P.host_weight(layer.weight, "bf16"), W0)


def test_weight_updates_without_input_grad(lib):
    from optimizer_step_weight_amd.autograd import FusedLinear
    _say("autograd input without grad")
    torch.manual_seed(1)
    layer = FusedLinear(128, 256, opt="sgd", hyper={"lr": 0.1}, seed=3)
    W0 = layer.weight.clone()
    x = torch.randn(64, 128, device="cuda").to(torch.bfloat16)      # no requires_grad
    layer(x).float().square().sum().backward()
    torch.cuda.synchronize()
    assert layer.step_count == 1 and not torch.equal(layer.weight, W0)


def _train(make_layers, steps, seed, lr):
    torch.manual_seed(seed)
    g = torch.Generator(device="cuda").manual_seed(seed)
    T, D, H = 512, 256, 512
    t1 = torch.randn(H, D, device="cuda", generator=g) / D ** 0.5
    t2 = torch.randn(D, H, device="cuda", generator=g) / H ** 0.5
    w1 = torch.randn(H, D, device="cuda", generator=g) / D ** 0.5
    w2 = torch.randn(D, H, device="cuda", generator=g) / H ** 0.5
    forward, params = make_layers(w1, w2)
    opt = torch.optim.AdamW(params, lr=lr, weight_decay=0.0) if params else None
    losses = []
    for _ in range(steps):
        x = torch.randn(T, D, device="cuda", generator=g)
        target = torch.relu(x @ t1.t()) @ t2.t()
        y = forward(x)
        loss = (y.float() - target).square().mean()
        if opt:
            opt.zero_grad(set_to_none=True)
        loss.backward()
        if opt:
            opt.step()
        losses.append(loss.detach().item())
    return np.array(losses)


def test_training_tracks_fp32_adamw(lib):
    from optimizer_step_weight_amd.autograd import FusedLinear
    _say("autograd training loop")
    lr, steps = 2e-3, 400

    def fused(w1, w2):
        l1 = FusedLinear(256, 512, opt="adamw", hyper={"lr": lr}, seed=11, weight=w1)
        l2 = FusedLinear(512, 256, opt="adamw", hyper={"lr": lr}, seed=12, weight=w2)
        return (lambda x: l2(torch.relu(l1(x.to(torch.bfloat16))))), []

    def reference(w1, w2):
        p1 = torch.nn.Parameter(w1.to(torch.bfloat16).float().clone())   # same starting values
        p2 = torch.nn.Parameter(w2.to(torch.bfloat16).float().clone())
        return (lambda x: torch.relu(x @ p1.t()) @ p2.t()), [p1, p2]

    a = _train(fused, steps, 5, lr)
    b = _train(reference, steps, 5, lr)
    sm = lambda z: np.convolve(z, np.ones(20) / 20, mode="valid")  # noqa: E731
    sa, sb = sm(a), sm(b)
    print(f"  loss: start {a[0]:.4f} / {b[0]:.4f}, end {sa[-1]:.4f} / {sb[-1]:.4f}, "
          f"max rel diff of 20-step means {np.max(np.abs(sa / sb - 1)):.3f}", flush=True)
    assert sa[-1] < 0.5 * a[0] and sb[-1] < 0.5 * b[0]           # both learn
    assert np.max(np.abs(sa / sb - 1)) < 0.15                     # and follow the same curve


@pytest.mark.parametrize("opt,state", [("adamw", "int8"), ("lion", "f32")])
def test_training_other_rules_learn(lib, opt, state):
    from optimizer_step_weight_amd.autograd import FusedLinear
    _say("autograd training", opt, state)
    lr = 2e-3 if opt == "adamw" else 2e-4

    def fused(w1, w2):
        l1 = FusedLinear(256, 512, opt=opt, hyper={"lr": lr}, state_dtype=state, seed=21, weight=w1)
        l2 = FusedLinear(512, 256, opt=opt, hyper={"lr": lr}, state_dtype=state, seed=22, weight=w2)
        return (lambda x: l2(torch.relu(l1(x.to(torch.bfloat16))))), []

    a = _train(fused, 300, 6, lr)
    sm = np.convolve(a, np.ones(20) / 20, mode="valid")
    print(f"  loss: start {a[0]:.4f}, end {sm[-1]:.4f}", flush=True)
    assert np.all(np.isfinite(a)) and sm[-1] < 0.7 * a[0]
