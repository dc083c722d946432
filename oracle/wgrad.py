"""Weight gradient, input gradient and the whole step (oracle; test infrastructure only).

FORGE explainer (gist.science), Technical Summary section 1 "The Problem":
the standard schedule forms the full weight gradient of a layer, stores it,
and only then runs the optimizer on it.  Section 2 "Core Mechanism": FORGE
instead accumulates, for one 128 x 128 tile of W at a time, the products of
the upstream gradient dY and the input X over all tokens, applies the
optimizer to that tile and discards the gradient; section 2 "Precision and
Fidelity": for element-wise rules both schedules give the same update, apart
from the floating-point order of the sum over tokens.

Here `step` is the two-phase definition (full dW, then the rule, then the
storage roundings) and `step_tiled` is the tile-by-tile consume-and-discard
schedule; tests check that they agree.  Section 5 "Significance and Claims"
(limitations): the input gradient must be read before the weight update, so
`dgrad` takes the weight as it was before the step.

Shapes: X[T, K], dY[T, N], W[N, K]; dW[n, k] = sum_t dY[t, n] * X[t, k];
dX[t, k] = sum_n dY[t, n] * W[n, k].
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import dynmap, numerics, optimizers

TILE = 128


def decode(fmt: str, data: np.ndarray, scale=None) -> np.ndarray:
    """Exact float64 value of a stored input tensor."""
    if fmt == "f32":
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return numerics.bf16_to_f64(data)
    if fmt == "fp8":
        return numerics.e4m3_to_f64(data) * np.float64(np.float32(scale))
    raise ValueError(fmt)


def decode_operand(op) -> np.ndarray:
    return decode(op.fmt, op.data, op.scale)


def wgrad(X64: np.ndarray, dY64: np.ndarray) -> np.ndarray:
    """dW = dY^T X in float64."""
    return dY64.T @ X64


def wgrad_abs(X64: np.ndarray, dY64: np.ndarray) -> np.ndarray:
    """sum_t |dY[t, n]| |X[t, k]|: the scale of the rounding error of any fp32 sum of dW."""
    return np.abs(dY64).T @ np.abs(X64)


def dgrad(dY64: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """dX = dY W in float64, with W as it was before the step."""
    return dY64 @ W64


def dgrad_bf16(dY64: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """dX stored as bf16 (round to nearest even from fp32, the kernel's precision)."""
    return numerics.bf16_rne(dgrad(dY64, W64).astype(np.float32))


def _decode_w(W, w_fmt):
    return numerics.bf16_to_f64(W) if w_fmt == "bf16" else np.asarray(W, np.float32).astype(np.float64)


def _codec(state_fmt):
    """The 8-bit moment map of a state format: "int8" linear absmax, "int8dyn" dynamic."""
    if state_fmt == "int8":
        return numerics
    if state_fmt == "int8dyn":
        return dynmap
    raise ValueError(state_fmt)


def _decode_state(st, state_fmt, signed):
    if st is None:
        return None
    if state_fmt == "f32":
        return np.asarray(st, np.float32).astype(np.float64)
    codes, scales = st
    return _codec(state_fmt).dequantize_block64(codes, scales, signed)


def decode_state(st, state_fmt, signed):
    """float64 values of a stored moment (fp32 array or (codes, scales))."""
    return _decode_state(st, state_fmt, signed)


def _encode_state(x64, state_fmt, signed):
    if x64 is None:
        return None
    if state_fmt == "f32":
        return x64.astype(np.float32)
    return _codec(state_fmt).quantize_block64(x64, signed)


def _zero_state(N, K, state_fmt, signed):
    if state_fmt == "f32":
        return np.zeros((N, K), np.float32)
    return (np.zeros((N, K), np.int8 if signed else np.uint8), np.zeros((N, K // numerics.BLOCK), np.float32))


def init_states(opt: str, N: int, K: int, state_fmt: str):
    """Zero moments for rule `opt` (None for a moment the rule does not keep)."""
    st = optimizers.STATES[opt]
    m = _zero_state(N, K, state_fmt, True) if "m" in st else None
    v = _zero_state(N, K, state_fmt, False) if "v" in st else None
    return m, v


def apply_rule(g, W, m, v, opt, hyper, t, seed, w_fmt, state_fmt, row0=0, col0=0, K_full=None):
    """Rule + storage roundings on one block of elements given its full gradient g.

    row0/col0 place the block inside the full [N, K_full] weight; the
    stochastic-rounding stream is keyed by the element's index in the full W.
    """
    rows, cols = g.shape
    K_full = cols if K_full is None else K_full
    W64 = _decode_w(W, w_fmt)
    m64 = _decode_state(m, state_fmt, True)
    v64 = _decode_state(v, state_fmt, False)
    W_new, m_new, v_new = optimizers.update(opt, hyper, t, g, W64, m64, v64)
    W32 = W_new.astype(np.float32)
    if w_fmt == "bf16":
        if col0 % 16 == 0 and cols % 16 == 0 and K_full % 16 == 0:
            bits = numerics.sr_bits_block(seed, t, row0, col0, rows, cols, K_full)
        else:
            idx = ((np.arange(rows, dtype=np.uint64)[:, None] + np.uint64(row0)) * np.uint64(K_full)
                   + np.arange(cols, dtype=np.uint64)[None, :] + np.uint64(col0))
            bits = numerics.sr_bits(seed, t, idx)
        W_st = numerics.sr_bf16(W32, bits)
    else:
        W_st = W32
    return dict(W=W_st, m=_encode_state(m_new, state_fmt, True), v=_encode_state(v_new, state_fmt, False),
                W32=W32, W64=W_new, m64=m_new, v64=v_new, g=g)


def step(X, dY, W, m, v, opt, hyper, t, seed, w_fmt, state_fmt, g: Optional[np.ndarray] = None) -> Dict:
    """Two-phase step: full dW, then the element-wise rule, then storage.

    X, dY are synth.Operand inputs; W is float32 or bf16 bits; m, v are
    float32 arrays or (codes, scales) pairs or None.
    """
    if g is None:
        g = wgrad(decode_operand(X), decode_operand(dY))
    return apply_rule(g, W, m, v, opt, hyper, t, seed, w_fmt, state_fmt)


def step_tiled(X, dY, W, m, v, opt, hyper, t, seed, w_fmt, state_fmt, tile: int = TILE) -> Dict:
    """Tile schedule: for each tile of W, its gradient, its update, then discard."""
    X64, dY64 = decode_operand(X), decode_operand(dY)
    N, K = (W.shape if not isinstance(W, tuple) else W[0].shape)
    out: Dict[str, np.ndarray] = {}
    for n0 in range(0, N, tile):
        for k0 in range(0, K, tile):
            n1, k1 = min(n0 + tile, N), min(k0 + tile, K)
            g = wgrad(X64[:, k0:k1], dY64[:, n0:n1])
            sub = lambda a: None if a is None else (
                (a[0][n0:n1, k0:k1], a[1][n0:n1, k0 // numerics.BLOCK:k1 // numerics.BLOCK])
                if isinstance(a, tuple) else a[n0:n1, k0:k1])
            r = apply_rule(g, W[n0:n1, k0:k1], sub(m), sub(v), opt, hyper, t, seed, w_fmt, state_fmt,
                           row0=n0, col0=k0, K_full=K)
            for key, val in r.items():
                if val is None:
                    out.setdefault(key, None)
                    continue
                if isinstance(val, tuple):
                    if key not in out:
                        out[key] = (np.empty((N, K), val[0].dtype), np.empty((N, K // numerics.BLOCK), np.float32))
                    out[key][0][n0:n1, k0:k1] = val[0]
                    out[key][1][n0:n1, k0 // numerics.BLOCK:k1 // numerics.BLOCK] = val[1]
                else:
                    if key not in out:
                        out[key] = np.empty((N, K), val.dtype)
                    out[key][n0:n1, k0:k1] = val
    return out
