"""Seeded synthetic inputs for the fused weight-gradient + optimizer step.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no arithmetic of the method itself: it only draws seeded random
numbers, encodes them into the storage formats the kernels read (fp32, bf16,
OCP fp8 e4m3 with a per-tensor scale) using PyTorch's own dtype conversions,
and describes the workloads (layer shapes, token counts, hyper-parameters).

Workloads follow the layer shapes the FORGE explainer pages (gist.science,
"FORGE: Fused On-Register Gradient Elimination for Memory-Efficient LLM
Training", Technical Summary section 4 "Experimental Results") train on:
Llama-3.1-8B and the Qwen3 family.  No dataset or trained weight is used; the
inputs are Gaussian with the standard deviations listed per workload.

Layout conventions (PyTorch nn.Linear): X[T, K] activations, dY[T, N] upstream
gradient, W[N, K] weight, all row-major and contiguous.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

# tensor ids used in the seed sequence
TID_X, TID_DY, TID_W = 0, 1, 2

OPTIMIZERS = ("adamw", "nadam", "radam", "lion", "rmsprop", "adagrad", "sgd", "sgd_momentum")


@dataclasses.dataclass(frozen=True)
class Hyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    wd_mode: int = 0           # 0 = the optimizer's customary mode, 1 = decoupled, 2 = coupled L2
    momentum: float = 0.9      # SGD-momentum
    alpha: float = 0.99        # RMSprop smoothing constant
    momentum_decay: float = 0.004  # NAdam momentum-decay schedule constant


def default_hyper(opt: str) -> Hyper:
    """Hyper-parameters of the optimizer sweep (textbook / library defaults)."""
    if opt == "adamw":
        return Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    if opt in ("nadam", "radam"):
        return Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    if opt == "lion":
        return Hyper(lr=1e-4, beta1=0.9, beta2=0.99, eps=0.0, weight_decay=0.01)
    if opt == "rmsprop":
        return Hyper(lr=1e-3, alpha=0.99, eps=1e-8)
    if opt == "adagrad":
        return Hyper(lr=1e-3, eps=1e-10)
    if opt == "sgd":
        return Hyper(lr=1e-3)
    if opt == "sgd_momentum":
        return Hyper(lr=1e-3, momentum=0.9)
    raise ValueError(opt)


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    N: int  # out features (rows of W)
    K: int  # in features (cols of W)


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    layers: Tuple[Layer, ...]
    T: int
    in_fmt: str          # 'f32' | 'bf16' | 'fp8'
    w_fmt: str           # 'f32' | 'bf16' (bf16 => stochastic rounding)
    state_fmt: str       # 'f32' | 'int8'
    optimizers: Tuple[str, ...]
    steps: int
    x_std: float
    dy_std: float
    w_std: float
    dgrad: bool = False
    hyper: Optional[Hyper] = None  # None => default_hyper(opt)

    def hyper_for(self, opt: str) -> Hyper:
        return self.hyper if self.hyper is not None else default_hyper(opt)


def _llama8b_block() -> Tuple[Layer, ...]:
    h, kv, f = 4096, 8 * 128, 14336
    return (Layer("q_proj", h, h), Layer("k_proj", kv, h), Layer("v_proj", kv, h),
            Layer("o_proj", h, h), Layer("gate_proj", f, h), Layer("up_proj", f, h),
            Layer("down_proj", h, f))


def _qwen3_14b_block() -> Tuple[Layer, ...]:
    h, kv, f = 5120, 8 * 128, 17408
    return (Layer("q_proj", 40 * 128, h), Layer("k_proj", kv, h), Layer("v_proj", kv, h),
            Layer("o_proj", h, 40 * 128), Layer("gate_proj", f, h), Layer("up_proj", f, h),
            Layer("down_proj", h, f))


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "single linear 256x256, fp32, T=512", (Layer("linear", 256, 256),), 512,
                "f32", "f32", "f32", ("adamw",), 3, 0.1, 0.1, 0.02,
                hyper=Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    2: Workload(2, "llama3.1-8b down_proj W[4096,14336], T=4096, bf16", (Layer("down_proj", 4096, 14336),),
                4096, "bf16", "bf16", "f32", ("adamw",), 5, 1.0, 1e-3, 0.02,
                hyper=Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    3: Workload(3, "llama3.1-8b decoder block (7 linears), T=8192, bf16, dgrad first", _llama8b_block(),
                8192, "bf16", "bf16", "f32", ("adamw",), 3, 1.0, 1e-3, 0.02, dgrad=True,
                hyper=Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    4: Workload(4, "qwen3-14b block (7 linears), T=4096, bf16, int8 block-64 moments", _qwen3_14b_block(),
                4096, "bf16", "bf16", "int8", ("adamw",), 10, 1.0, 1e-3, 0.02,
                hyper=Hyper(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)),
    5: Workload(5, "optimizer sweep W[4096,4096], T=16384, bf16 and fp8 inputs", (Layer("linear", 4096, 4096),),
                16384, "bf16", "bf16", "f32", OPTIMIZERS, 8, 1.0, 1e-3, 0.02),
}


def sr_seed(cfg: int, layer: int) -> int:
    """Per-layer stochastic-rounding seed."""
    return 0x5EED0000 + 256 * cfg + layer


def rng_for(cfg: int, step: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, step, layer, tensor_id]))


# ----------------------------------------------------------------------------- encoders
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) via PyTorch; returns uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp8_e4m3(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """Per-tensor scaled OCP e4m3 encoding via PyTorch: s = amax/448, codes = e4m3(x/s)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    y = np.clip(x / s, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


@dataclasses.dataclass
class Operand:
    """One input tensor in its storage format."""
    fmt: str                 # 'f32' | 'bf16' | 'fp8'
    data: np.ndarray         # float32 | uint16 bits | uint8 codes
    scale: Optional[np.float32] = None  # fp8 per-tensor scale


def encode(x: np.ndarray, fmt: str) -> Operand:
    if fmt == "f32":
        return Operand("f32", np.ascontiguousarray(x, dtype=np.float32))
    if fmt == "bf16":
        return Operand("bf16", to_bf16_bits(x))
    if fmt == "fp8":
        c, s = to_fp8_e4m3(x)
        return Operand("fp8", c, s)
    raise ValueError(fmt)


def gaussian(cfg: int, step: int, layer: int, tensor_id: int, shape, std: float) -> np.ndarray:
    g = rng_for(cfg, step, layer, tensor_id)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def layer_inputs(w: Workload, step: int, layer_idx: int, in_fmt: Optional[str] = None,
                 T: Optional[int] = None) -> Tuple[Operand, Operand]:
    """Fresh seeded X[T,K] and dY[T,N] for one step of one layer."""
    L = w.layers[layer_idx]
    T = w.T if T is None else T
    fmt = in_fmt or w.in_fmt
    X = gaussian(w.cfg, step, layer_idx, TID_X, (T, L.K), w.x_std)
    dY = gaussian(w.cfg, step, layer_idx, TID_DY, (T, L.N), w.dy_std)
    return encode(X, fmt), encode(dY, fmt)


def layer_weight(w: Workload, layer_idx: int) -> np.ndarray:
    """Initial W[N,K] in the workload's weight format (float32 or bf16 bits)."""
    L = w.layers[layer_idx]
    W = gaussian(w.cfg, 0, layer_idx, TID_W, (L.N, L.K), w.w_std)
    return W if w.w_fmt == "f32" else to_bf16_bits(W)


# ----------------------------------------------------------------------------- small / exact cases
def gaussian_case(seed: int, T: int, N: int, K: int, fmt: str, x_std=1.0, dy_std=1e-3):
    g = np.random.default_rng(np.random.SeedSequence([99, seed]))
    X = (g.standard_normal((T, K), dtype=np.float32) * np.float32(x_std))
    dY = (g.standard_normal((T, N), dtype=np.float32) * np.float32(dy_std))
    return encode(X, fmt), encode(dY, fmt)


def integer_case(seed: int, T: int, N: int, K: int, fmt: str):
    """Inputs on a dyadic grid whose fp32 partial sums are exact in any order.

    X in {-1, -0.75, ..., 1}, dY in {-3..3} * 2^-10.  Every product is a multiple
    of 2^-12 and |sum| <= T * 3 * 2^-10, so for T <= 2^16 every partial sum has
    fewer than 24 significant bits.  For fp8 the values are stored as e4m3 codes
    of {-4..4}/4 and {-3..3}/4 with power-of-two scales 1 and 2^-8.
    """
    assert T <= 65536
    g = np.random.default_rng(np.random.SeedSequence([77, seed]))
    xi = g.integers(-4, 5, size=(T, K)).astype(np.float32)
    di = g.integers(-3, 4, size=(T, N)).astype(np.float32)
    if fmt == "fp8":
        cx = torch.from_numpy(xi / 4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        cd = torch.from_numpy(di / 4).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return Operand("fp8", cx, np.float32(1.0)), Operand("fp8", cd, np.float32(2.0 ** -8))
    return encode(xi * np.float32(0.25), fmt), encode(di * np.float32(2.0 ** -10), fmt)


def random_weight(seed: int, N: int, K: int, fmt: str, std=0.02) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([55, seed]))
    W = g.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return W if fmt == "f32" else to_bf16_bits(W)
