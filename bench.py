"""Benchmark of the fused weight-gradient + AdamW step on one MI355X.

Workload (one step = one fused launch = the whole hot path for one linear layer): the
Llama-3.1-8B down_proj shape W[N=4096, K=14336] bf16, X[T=4096, 14336] ~ N(0,1) bf16,
dY[4096, 4096] ~ N(0, 1e-3) bf16, fp32 m and v, AdamW (lr 1e-3, betas 0.9/0.999, eps 1e-8,
wd 0.01 decoupled), bf16 weight write-back with stochastic rounding.  Inputs are synthetic
and seeded; two input batches alternate so that consecutive steps do not re-read one batch
from the last-level cache.

Prints one JSON line: throughput in TFLOP/s (2 T N K per step), the roofline of the fused
kernel, the CPU oracle's rate on a bounded sample of the same step, and side numbers (the
unfused GEMM + optimizer path, dgrad, peak memory).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu] [--no-extra]
       python bench.py --copy-calibration      (plain copy kernel for HBM counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "fused wgrad+AdamW TFLOP/s and % bf16 MFMA peak (8B down_proj, T=4096)"
PMC_FILE = os.path.join(ROOT, "profiles", "fused_adamw_down_proj_T4096_hbm_counters.json")


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "optimizer_step_weight_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter runs, if the kernels have not changed since."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(rows: int):
    """The oracle (fp64 two-phase step) on `rows` rows of W with the full T and K."""
    import numpy as np

    import synth
    from oracle import wgrad
    w = synth.WORKLOADS[2]
    L = w.layers[0]
    X, dY = synth.layer_inputs(w, 1, 0)
    W = synth.layer_weight(w, 0)[:rows]
    dYs = synth.Operand("bf16", np.ascontiguousarray(dY.data[:, :rows]))
    m, v = wgrad.init_states("adamw", rows, L.K, "f32")
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    wgrad.step(X, dYs, W, m, v, "adamw", w.hyper, 1, synth.sr_seed(2, 0), "bf16", "f32")
    dt = time.perf_counter() - t0
    flop = 2.0 * w.T * rows * L.K
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {L.N} rows of W (full T={w.T}, K={L.K}): fp64 dW by BLAS, fp64 AdamW, "
                      f"Philox stochastic rounding; {dt:.1f} s"}


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def run_one(a, forge, batches, W, m, v, h, seed, T, N, K):
    """Time one kernel of the headline shape alone (warmup + steps launches)."""
    import torch
    dW = torch.empty((N, K), dtype=torch.float32, device="cuda") if a.kernel in ("gemm", "optimizer") else None
    dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda") if a.kernel == "dgrad" else None
    if a.kernel == "optimizer":
        dW.normal_(0, 0.06)

    def once(t):
        Xd, Dd = batches[t % 2]
        if a.kernel == "fused":
            forge.wgrad_step(Xd, Dd, W, m, v, opt="adamw", hyper=h, step=t, seed=seed)
        elif a.kernel == "gemm":
            forge.wgrad_gemm(Xd, Dd, dW)
        elif a.kernel == "optimizer":
            forge.optimizer_step(dW, W, m, v, opt="adamw", hyper=h, step=t, seed=seed)
        else:
            forge.dgrad(Dd, W, dX)
    for t in range(1, a.warmup + 1):
        once(t)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for t in range(a.warmup + 1, a.warmup + a.steps + 1):
        once(t)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps
    flop = 2.0 * T * N * K
    print(json.dumps({"kernel": a.kernel, "us_per_launch": round(ms * 1e3, 2),
                      "tflops": round(flop / (ms * 1e-3) / 1e12, 1) if a.kernel != "optimizer" else None}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kernel", choices=["fused", "gemm", "optimizer", "dgrad"], default=None,
                    help="run only this kernel of the headline shape (for profiler runs); prints its time")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {a.gpus} requested). The fused step shards "
              "by whole weight tiles with no exchange; see DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import optimizer_step_weight_amd as forge
    import synth

    if a.copy_calibration:
        copy_calibration()
        return
    if not os.path.exists(forge.LIB_PATH):
        from optimizer_step_weight_amd import _build
        _build.build(verbose=False)
    torch.cuda.set_device(0)
    forge.device_check(0)

    w = synth.WORKLOADS[2]
    L = w.layers[0]
    T, N, K = w.T, L.N, L.K
    h = w.hyper
    seed = synth.sr_seed(2, 0)
    print(f"[bench] generating inputs T={T} N={N} K={K}", file=sys.stderr, flush=True)
    batches = []
    for s in (1, 2):
        X, dY = synth.layer_inputs(w, s, 0)
        batches.append((torch.from_numpy(X.data.view(np.int16)).cuda().view(torch.bfloat16),
                        torch.from_numpy(dY.data.view(np.int16)).cuda().view(torch.bfloat16)))
    W = torch.from_numpy(synth.layer_weight(w, 0).view(np.int16)).cuda().view(torch.bfloat16)
    m = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    v = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(t):
        Xd, Dd = batches[t % 2]
        forge.wgrad_step(Xd, Dd, W, m, v, opt="adamw", hyper=h, step=t, seed=seed)

    if a.kernel is not None:
        run_one(a, forge, batches, W, m, v, h, seed, T, N, K)
        return

    t = 0
    for _ in range(a.warmup):
        t += 1
        step(t)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(a.steps):
        t += 1
        step(t)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps
    fused_peak_extra = torch.cuda.max_memory_allocated() - base_alloc
    flop = 2.0 * T * N * K
    tflops = flop / (ms * 1e-3) / 1e12
    print(f"[bench] fused step {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    extra = {"fused_peak_extra_bytes": int(fused_peak_extra)}
    if not a.no_extra:
        # unfused two-phase baseline: dW GEMM to HBM, then the optimizer kernel
        torch.cuda.reset_peak_memory_stats()
        base_alloc = torch.cuda.memory_allocated()
        dW = torch.empty((N, K), dtype=torch.float32, device="cuda")

        def unfused(t):
            Xd, Dd = batches[t % 2]
            forge.wgrad_gemm(Xd, Dd, dW)
            forge.optimizer_step(dW, W, m, v, opt="adamw", hyper=h, step=t, seed=seed)
        for _ in range(2):
            t += 1
            unfused(t)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        gemm_ms = opt_ms = 0.0
        for _ in range(a.steps):
            t += 1
            Xd, Dd = batches[t % 2]
            e[0].record()
            forge.wgrad_gemm(Xd, Dd, dW)
            e[1].record()
            forge.optimizer_step(dW, W, m, v, opt="adamw", hyper=h, step=t, seed=seed)
            e[2].record()
            torch.cuda.synchronize()
            gemm_ms += e[0].elapsed_time(e[1])
            opt_ms += e[1].elapsed_time(e[2])
        unf_peak_extra = torch.cuda.max_memory_allocated() - base_alloc
        del dW
        gemm_ms /= a.steps
        opt_ms /= a.steps
        # dgrad on the same layer (dX = dY W), bf16 out
        dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            forge.dgrad(batches[0][1], W, dX)
        ev0.record()
        for _ in range(a.steps):
            forge.dgrad(batches[0][1], W, dX)
        ev1.record()
        torch.cuda.synchronize()
        dg_ms = ev0.elapsed_time(ev1) / a.steps
        del dX
        extra.update({
            "unfused_ms": round(gemm_ms + opt_ms, 4), "unfused_gemm_ms": round(gemm_ms, 4),
            "unfused_optimizer_ms": round(opt_ms, 4), "fused_speedup_vs_unfused": round((gemm_ms + opt_ms) / ms, 3),
            "unfused_peak_extra_bytes": int(unf_peak_extra), "dgrad_ms": round(dg_ms, 4),
            "dgrad_tflops": round(flop / (dg_ms * 1e-3) / 1e12, 1),
            "optimizer_kernel_hbm_gbs": round(N * K * (4 + 4 + 8 + 8) / (opt_ms * 1e-3) / 1e9, 1),
        })
        print(f"[bench] unfused {gemm_ms * 1e3:.1f} + {opt_ms * 1e3:.1f} us; dgrad {dg_ms * 1e3:.1f} us",
              file=sys.stderr, flush=True)

    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic()}
    cpu = None
    if not a.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(a.cpu_rows)
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded Gaussian, down_proj shapes)",
        "config": {"workload": "llama3.1-8b down_proj wgrad+AdamW step: W[4096,14336] bf16 (SR), fp32 m/v, "
                               "X[4096,14336], dY[4096,4096] bf16", "T": T, "N": N, "K": K,
                   "optimizer": "adamw", "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
