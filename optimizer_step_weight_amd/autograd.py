"""PyTorch autograd integration: a linear layer whose backward pass updates its own weight.

FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": the weight
gradient of a layer is consumed tile by tile by the optimizer and never stored.  In a PyTorch
model that means the layer's backward does the update: `FusedLinear.backward` calls the
library's `linear_backward_step`, which computes the input gradient dX = dY W with the weight as
it was (section 5 "Significance and Claims": the input gradient must be read before the update),
then runs the fused weight-gradient + optimizer step on W and its moments in place.  The layer
returns no weight gradient, so no optimizer object and no `.grad` buffer exist for it.

Limits the method imposes (section 5): a weight used by several consumers in one step (tied
embeddings, shared layers) cannot be updated by one of them, and non-element-wise steps such as
global gradient-norm clipping cannot see this weight's gradient.  Each forward of a layer must be
followed by exactly one backward before the next forward.

All arithmetic runs in the library's kernels; this module only marshals tensors.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import linear_backward_step, wgrad_step

_STATES = {"adamw": "mv", "nadam": "mv", "radam": "mv", "lion": "m", "rmsprop": "v", "adagrad": "v",
           "sgd": "", "sgd_momentum": "m"}


class _LinearStep(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2d, anchor, layer):
        ctx.layer = layer
        ctx.save_for_backward(x2d)
        return x2d @ layer.weight.t()

    @staticmethod
    def backward(ctx, dy):
        (x2d,) = ctx.saved_tensors
        layer = ctx.layer
        dy = dy.contiguous()
        if dy.dtype != layer.weight.dtype:
            dy = dy.to(layer.weight.dtype)
        layer.step_count += 1
        kw = dict(opt=layer.opt, hyper=layer.hyper, step=layer.step_count, seed=layer.seed,
                  m_scale=layer.m_scale, v_scale=layer.v_scale)
        if ctx.needs_input_grad[0]:
            dx = torch.empty_like(x2d)
            linear_backward_step(x2d, dy, layer.weight, dx, layer.m, layer.v, **kw)
        else:
            dx = None
            wgrad_step(x2d, dy, layer.weight, layer.m, layer.v, **kw)
        return dx, None, None


class FusedLinear(torch.nn.Module):
    """y = x W^T with W [out_features, in_features] bf16 (stochastic rounding on update) and the
    rule's moments on the device.  `in_features` and `out_features` must be multiples of 128.

    opt: one of adamw, nadam, radam, lion, rmsprop, adagrad, sgd, sgd_momentum.
    hyper: dict or object with the rule's hyper-parameters (defaults: lr 1e-3, betas 0.9 /
        0.999, eps 1e-8, no weight decay).
    state_dtype: "f32" or "int8" (block-64 absmax moments).
    seed: the stochastic-rounding key of this layer (give every layer its own).
    """

    def __init__(self, in_features: int, out_features: int, *, opt: str = "adamw",
                 hyper=None, state_dtype: str = "f32", seed: int = 0,
                 weight: Optional[torch.Tensor] = None, device="cuda"):
        super().__init__()
        if in_features % 128 or out_features % 128:
            raise ValueError("in_features and out_features must be multiples of 128")
        if opt not in _STATES:
            raise ValueError(f"unknown rule {opt!r}")
        self.in_features, self.out_features = in_features, out_features
        self.opt, self.seed = opt, int(seed)
        # hyper-parameters: any object or dict with lr, beta1, beta2, eps, weight_decay, wd_mode,
        # momentum, alpha, momentum_decay; missing fields take the library's defaults
        self.hyper = hyper if hyper is not None else {}
        if weight is None:
            weight = torch.randn(out_features, in_features, device=device) * (1.0 / in_features ** 0.5)
        self.register_buffer("weight", weight.to(device=device, dtype=torch.bfloat16).contiguous())
        shape = (out_features, in_features)
        nblk = out_features * in_features // 64
        st = _STATES[opt]

        def state(signed: bool, needed: bool):
            if not needed:
                return None, None
            if state_dtype == "f32":
                return torch.zeros(shape, device=device), None
            if state_dtype == "int8":
                return (torch.zeros(shape, dtype=torch.int8 if signed else torch.uint8, device=device),
                        torch.zeros(nblk, device=device))
            raise ValueError(f"unknown state dtype {state_dtype!r}")
        m, ms = state(True, "m" in st)
        v, vs = state(False, "v" in st)
        self.register_buffer("m", m)
        self.register_buffer("m_scale", ms)
        self.register_buffer("v", v)
        self.register_buffer("v_scale", vs)
        self.step_count = 0
        # a zero-size leaf that requires grad, so that backward runs (and the weight is updated)
        # even when the layer's input needs no gradient
        self._anchor = torch.nn.Parameter(torch.empty(0, device=device), requires_grad=True)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2d = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        y = _LinearStep.apply(x2d, self._anchor, self)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, opt={self.opt}"
