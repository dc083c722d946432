"""Drift of the Qwen3-14B block with int8 moments against a free-running float64 ideal.

FORGE explainer (gist.science), Technical Summary section 2 "Precision and Fidelity" (int8
states in blocks of 64, stochastic rounding of the bf16 weight) and section 3 (full-precision
fidelity at low precision); section 4 reports training that tracks fused AdamW.  With no data
or weights here, the check is on the optimizer trajectory itself: every linear of the block
(T = 4096, AdamW, 10 steps, fresh seeded Gaussian X and dY every step) runs free on the device
over the whole layer in several storage variants, from the same bf16 W0:

  int8-sr      int8 block-64 moments (linear absmax map), stochastic rounding (the workload)
  int8-rne     int8 moments, nearest-even rounding (control: what stochastic rounding adds)
  f32-sr       fp32 moments, stochastic rounding (control: what int8 moments cost)
  dyn8-sr      int8 block-64 moments in the dynamic 8-bit map, stochastic rounding

Blocks of 2048 (the block size of common 8-bit optimizers, which the pages contrast with 64) span
sixteen tiles of a row, so a tile-fused kernel cannot form them; the oracle runs those variants
on the sampled rows instead, with the same stochastic-rounding stream:

  int8-b2048-sr, dyn8-b2048-sr   (oracle only)

and the oracle follows the same rows in the ideal: float64 weight and moments, no quantisation,
no rounding.  Per step it reports, with dW = W_t - W_0 on the sampled rows,
  rel   = ||dW_dev - dW_ideal|| / ||dW_ideal||
  bias  = mean(dW_dev - dW_ideal) / mean|dW_ideal|   (mean signed error)
The bounds asserted are loose (a broken codec or rounding moves them by orders of magnitude);
the numbers themselves are the report.  With FORGE_REPORT_DIR set, they are also written there
as drift_qwen3_14b_block.json.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import dynmap, numerics, optimizers, wgrad
from tests import parity as P

pytestmark = pytest.mark.gpu

VARIANTS = {"int8-sr": ("int8", True), "int8-rne": ("int8", False), "f32-sr": ("f32", True),
            "dyn8-sr": ("int8dyn", True)}
HOST_VARIANTS = {"int8-b2048-sr": numerics, "dyn8-b2048-sr": dynmap}
STEPS = 10
_REPORT = {}


@pytest.fixture(scope="module")
def lib():
    import optimizer_step_weight_amd as forge
    if not os.path.exists(forge.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    forge.device_check(0)
    return forge


def _rows(N):
    """32 sampled rows: 4 at each of 8 places spread over the layer."""
    return np.concatenate([np.arange(r, r + 4) for r in np.linspace(0, N - 4, 8).astype(int) // 4 * 4])


@pytest.mark.parametrize("li", range(7), ids=[L.name for L in synth.WORKLOADS[4].layers])
def test_qwen3_block_drift_against_float64_ideal(lib, li):
    w = synth.WORKLOADS[4]
    L = w.layers[li]
    N, K, T = L.N, L.K, w.T
    h = w.hyper
    seed = synth.sr_seed(4, li)
    W0 = synth.layer_weight(w, li)
    rows = _rows(N)
    devs = {}
    for name, (state_fmt, _sr) in VARIANTS.items():
        m, v = wgrad.init_states("adamw", N, K, state_fmt)
        devs[name] = P.DeviceStep(W0, m, v, "bf16", state_fmt)
    W0r = numerics.bf16_to_f64(W0[rows])
    Wi, mi, vi = W0r.copy(), np.zeros_like(W0r), np.zeros_like(W0r)
    # oracle-only variants: bf16 weight bits and block-2048 moments (codes, scales) of the rows
    host = {name: [W0[rows].copy(), None, None] for name in HOST_VARIANTS}
    report = []
    for t in range(1, STEPS + 1):
        print(f"[case] drift {L.name} [{N}x{K}] step {t}", flush=True)
        X, dY = synth.layer_inputs(w, t, li)
        Xd, _ = P.dev_operand(X)
        Dd, _ = P.dev_operand(dY)
        for name, (state_fmt, sr) in VARIANTS.items():
            d = devs[name]
            lib.wgrad_step(Xd, Dd, d.W, d.m, d.v, opt="adamw", hyper=h, step=t, seed=seed, m_scale=d.ms,
                           v_scale=d.vs, sr=sr, state_map=d.state_map)
        torch.cuda.synchronize()
        del Xd, Dd
        g = wgrad.decode_operand(dY)[:, rows].T @ wgrad.decode_operand(X)
        Wi, mi, vi = optimizers.update("adamw", h, t, g, Wi, mi, vi)
        dWi = Wi - W0r
        row = {"step": t}
        for name, codec in HOST_VARIANTS.items():
            Wb, mq, vq = host[name]
            m64 = np.zeros_like(g) if mq is None else codec.dequantize_blocks(*mq, True, 2048)
            v64 = np.zeros_like(g) if vq is None else codec.dequantize_blocks(*vq, False, 2048)
            Wn, mn, vn = optimizers.update("adamw", h, t, g, numerics.bf16_to_f64(Wb), m64, v64)
            bits = np.stack([numerics.sr_bits_block(seed, t, int(r), 0, 1, K, K)[0] for r in rows])
            host[name] = [numerics.sr_bf16(Wn.astype(np.float32), bits), codec.quantize_blocks(mn, True, 2048),
                          codec.quantize_blocks(vn, False, 2048)]
            e = numerics.bf16_to_f64(host[name][0]) - W0r - dWi
            row[name] = {"rel": float(np.linalg.norm(e) / np.linalg.norm(dWi)),
                         "bias": float(np.mean(e) / np.mean(np.abs(dWi)))}
        for name, d in devs.items():
            dWd = numerics.bf16_to_f64(P.host_weight(d.W[torch.from_numpy(rows).cuda()], "bf16")) - W0r
            e = dWd - dWi
            row[name] = {"rel": float(np.linalg.norm(e) / np.linalg.norm(dWi)),
                         "bias": float(np.mean(e) / np.mean(np.abs(dWi)))}
        report.append(row)
        print("  " + "; ".join(f"{n}: rel {row[n]['rel']:.3e} bias {row[n]['bias']:+.2e}"
                               for n in list(VARIANTS) + list(HOST_VARIANTS)), flush=True)
    _REPORT[L.name] = {"N": N, "K": K, "T": T, "rows": len(rows), "steps": report}
    out = os.environ.get("FORGE_REPORT_DIR")
    if out:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "drift_qwen3_14b_block.json"), "w") as f:
            json.dump(_REPORT, f, indent=1)
    for row in report:
        for name in list(VARIANTS) + list(HOST_VARIANTS):
            assert row[name]["rel"] < 0.5, f"{L.name} {name} step {row['step']}: rel drift {row[name]['rel']:.3e}"
        for name in VARIANTS:
            if VARIANTS[name][1]:
                assert abs(row[name]["bias"]) < 0.02, f"{L.name} {name} step {row['step']}: bias {row[name]['bias']:.3e}"
