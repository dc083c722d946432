"""Benchmark of the fused weight-gradient + AdamW step on one MI355X.

Workload (one step = one fused launch = the whole hot path for one linear layer): the
Llama-3.1-8B down_proj shape W[N=4096, K=14336] bf16, X[T=4096, 14336] ~ N(0,1) bf16,
dY[4096, 4096] ~ N(0, 1e-3) bf16, fp32 m and v, AdamW (lr 1e-3, betas 0.9/0.999, eps 1e-8,
wd 0.01 decoupled), bf16 weight write-back with stochastic rounding.  Inputs are synthetic
and seeded; two input batches alternate so that consecutive steps do not re-read one batch
from the last-level cache.

Prints one JSON line: throughput in TFLOP/s (2 T N K per step) over `steps` fused steps run
back to back after `warmup` untimed ones, the roofline of the fused kernel, the CPU oracle's
rate on a bounded sample of the same step, and in "extra": per-step p10/p50/p90 warm and cold
(L2 and last-level cache flushed before each step), the unfused GEMM + optimizer path (same
protocol) and hipBLASLt's GEMM for the same product as context, dgrad, peak memory, and the
other workloads (the 7-linear Llama-3.1-8B block with dgrad, the Qwen3-14B block with int8
moments, the 8-rule sweep with bf16 and fp8 inputs).

Before the warmup steps, untimed fused steps run for --settle-ms (default 150 ms): under
sustained load the GPU's power management overshoots for its first ~20 launches before it
settles, and the timed steps are meant to measure the steady state (the settle phase's
per-launch times are reported in "extra").

Usage: python bench.py [--gpus 1] [--steps 30] [--warmup 20] [--settle-ms 150] [--no-cpu] [--no-extra]
       python bench.py --copy-calibration      (plain copy kernel for HBM counter scaling)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "fused wgrad+AdamW TFLOP/s and % bf16 MFMA peak (8B down_proj, T=4096)"
# the moments each update rule keeps (which state buffers a call passes)
RULE_STATES = {"adamw": "mv", "nadam": "mv", "radam": "mv", "lion": "m", "rmsprop": "v", "adagrad": "v",
               "sgd": "", "sgd_momentum": "m"}
PMC_FILE = os.path.join(ROOT, "profiles", "fused_adamw_down_proj_T4096_hbm_counters.json")


def source_hash() -> str:
    """The library's build id for the sources under ROOT (HBM counters are valid only for them)."""
    from optimizer_step_weight_amd import _build
    return _build.source_hash(ROOT)


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


def cpu_baseline(rows: int, steps: int):
    """The oracle (fp64 two-phase step) on `rows` rows of W with the full T and K, `steps` times."""
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
    try:
        blas = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except (TypeError, AttributeError):
        blas = "unknown"
    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        r = wgrad.step(X, dYs, W, m, v, "adamw", w.hyper, t, synth.sr_seed(2, 0), "bf16", "f32")
        W, m, v = r["W"], r["m"], r["v"]
    dt = time.perf_counter() - t0
    flop = 2.0 * w.T * rows * L.K * steps
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} steps on {rows} of {L.N} rows of W (full T={w.T}, K={L.K}; one input batch): "
                      f"fp64 dW by BLAS ({blas}), fp64 AdamW, Philox stochastic rounding; {dt:.1f} s"}


def cpu_oracle_other_workloads(rows: int = 128):
    """The oracle's throughput on bounded samples of the other workloads (host cores): every
    layer or case with its full T and K and the first `rows` rows of W (their dY columns), one
    step; for the Llama block also dgrad on the first `rows` tokens with the whole W.  Input
    generation is outside the timed regions."""
    import numpy as np

    import synth
    from oracle import wgrad
    res = {}
    for cfg in (3, 4, 5):
        w = synth.WORKLOADS[cfg]
        flop = secs = 0.0
        cases = [(li, opt, fmt) for li in range(len(w.layers)) for fmt in ((w.in_fmt,) if cfg != 5 else ("bf16", "fp8"))
                 for opt in w.optimizers]
        inputs = {}
        for li, opt, fmt in cases:
            L = w.layers[li]
            if (li, fmt) not in inputs:
                inputs.clear()
                inputs[(li, fmt)] = synth.layer_inputs(w, 1, li, in_fmt=fmt), synth.layer_weight(w, li)
            (X, dY), W = inputs[(li, fmt)]
            dYs = synth.Operand(dY.fmt, np.ascontiguousarray(dY.data[:, :rows]), dY.scale)
            m, v = wgrad.init_states(opt, rows, L.K, w.state_fmt)
            t0 = time.perf_counter()
            wgrad.step(X, dYs, W[:rows], m, v, opt, w.hyper_for(opt), 1, synth.sr_seed(cfg, li), w.w_fmt, w.state_fmt)
            secs += time.perf_counter() - t0
            flop += 2.0 * w.T * rows * L.K
            if w.dgrad:
                dYt = wgrad.decode_operand(dY)[:rows]
                t0 = time.perf_counter()
                wgrad.dgrad_bf16(dYt, wgrad.decode("bf16", W))
                secs += time.perf_counter() - t0
                flop += 2.0 * rows * L.N * L.K
        res[w.name] = {"value": round(flop / secs / 1e12, 6), "unit": "TFLOP/s", "seconds": round(secs, 2),
                       "sample": f"{len(cases)} layer/rule cases, {rows} rows of W each (full T={w.T} and K), one step"
                                 + (f"; dgrad on {rows} tokens with the whole W" if w.dgrad else "")}
    return {"cores": len(os.sched_getaffinity(0)), "kind": "oracle", "workloads": res}


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


def pctl(ms_list):
    """p10 / p50 / p90 of per-step times (ms) in microseconds."""
    import numpy as np
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"p10": round(float(np.percentile(a, 10)), 1), "p50": round(float(np.percentile(a, 50)), 1),
            "p90": round(float(np.percentile(a, 90)), 1)}


class Timer:
    """Per-launch times on the current stream: warm (back to back, one event between launches)
    and cold (L2 and the last-level cache flushed by a 512 MiB write before each launch,
    outside the timed region)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.scratch = None

    def warm(self, fn, reps):
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(reps):
            fn(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
        return ev[0].elapsed_time(ev[reps]) / reps, per

    def cold(self, fn, reps):
        torch = self.torch
        if self.scratch is None:
            self.scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = []
        for i in range(reps):
            self.scratch.fill_(i & 0xFF)
            torch.cuda.synchronize()
            e0.record()
            fn(i)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1))
        return per


def clock_during(forge, fn, reps, seconds):
    """Average shader clock (MHz) while `fn` runs `reps` times back to back on the current
    stream: a one-wave sampler on a second stream (default priority) spans the first `seconds`
    of the run, measuring shader-clock cycles against the constant-rate real-time counter."""
    import torch
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    forge.clock_sample(seconds, out, stream=side.cuda_stream)
    for i in range(reps):
        fn(i)
    torch.cuda.synchronize()
    cycles, ticks = (int(x) for x in out.tolist())
    hz = forge.realtime_hz()
    return round(cycles / (ticks / hz) / 1e6, 1) if ticks > 0 and hz > 0 else None


WORKLOAD_PARTS = ("single", "llama", "qwen", "sweep")


def workload_timings(forge, timer, reps, parts=WORKLOAD_PARTS):
    """The other workloads' steps on device-generated Gaussian inputs of the same shapes and scales:
    the single fp32 linear (W[256, 256], T = 512), the 7-linear Llama-3.1-8B block (dgrad then the
    fused step per layer, T = 8192), the Qwen3-14B block with int8 moments (T = 4096; per layer
    also with fp32 moments and the contraction alone), and the 8-rule sweep on W[4096, 4096]
    (T = 16384) with bf16 and fp8 e4m3 inputs (and the contraction alone in each).  Each also
    times its unfused counterpart (GEMM to an fp32 dW, then the optimizer kernel)."""
    import torch

    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)

    def randn(shape, std, dtype=torch.bfloat16):
        return (torch.randn(shape, device="cuda", generator=gen) * std).to(dtype)

    def fp8(x):
        s = (x.float().abs().max() / 448.0).reshape(1)
        return (x.float() / s).clamp(-448, 448).to(torch.float8_e4m3fn), s

    def p50_of(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        times = []
        for r in range(n + 2):
            torch.cuda.synchronize()
            ev[0].record()
            fn(r)
            ev[1].record()
            torch.cuda.synchronize()
            if r >= 2:
                times.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return round(float(sorted(times)[len(times) // 2]), 1)

    out = {}
    if "single" in parts:
        out.update(_single_fp32(forge, reps, p50_of))
    if "llama" in parts:
        out.update(_llama_block(forge, reps, randn))
    if "qwen" in parts:
        out.update(_qwen_block(forge, reps, randn, p50_of))
    if "sweep" in parts:
        out.update(_sweep(forge, reps, randn, fp8, p50_of))
    return out


def _llama_block(forge, reps, randn):
    import torch

    import synth
    out = {}
    # Llama-3.1-8B block: dgrad + fused AdamW step per linear
    w = synth.WORKLOADS[3]
    T = w.T
    layers = []
    for L in w.layers:
        layers.append(dict(name=L.name, N=L.N, K=L.K, X=randn((T, L.K), w.x_std), dY=randn((T, L.N), w.dy_std),
                           W=randn((L.N, L.K), w.w_std), m=torch.zeros((L.N, L.K), device="cuda"),
                           v=torch.zeros((L.N, L.K), device="cuda"),
                           dX=torch.empty((T, L.K), dtype=torch.bfloat16, device="cuda")))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)]
    per_layer = [[] for _ in layers]
    block = []
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    for r in range(reps + 2):
        if r == 1:  # the peak memory of one whole fused block step (the first iteration)
            torch.cuda.synchronize()
            fused_extra = torch.cuda.max_memory_allocated() - base
        torch.cuda.synchronize()
        ev[0].record()
        for i, d in enumerate(layers):
            forge.linear_backward_step(d["X"], d["dY"], d["W"], d["dX"], d["m"], d["v"], opt="adamw", hyper=w.hyper,
                                       step=r + 1, seed=synth.sr_seed(3, i))
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r >= 2:
            block.append(ev[0].elapsed_time(ev[-1]))
            for i in range(len(layers)):
                per_layer[i].append(ev[i].elapsed_time(ev[i + 1]))
    flop = sum(4.0 * T * d["N"] * d["K"] for d in layers)
    b50 = pctl(block)["p50"]
    # the unfused block: dgrad, the GEMM into one fp32 dW buffer shared by the layers (the
    # smallest gradient memory an unfused step can have; all 7 alive together would need
    # 832 MiB), then the optimizer kernel
    dW = torch.empty(max(d["N"] * d["K"] for d in layers), dtype=torch.float32, device="cuda")
    ub = []
    for r in range(reps + 2):
        torch.cuda.synchronize()
        ev[0].record()
        for i, d in enumerate(layers):
            g = dW[:d["N"] * d["K"]].view(d["N"], d["K"])
            forge.dgrad(d["dY"], d["W"], d["dX"])
            forge.wgrad_gemm(d["X"], d["dY"], g)
            forge.optimizer_step(g, d["W"], d["m"], d["v"], opt="adamw", hyper=w.hyper, step=reps + 3 + r,
                                 seed=synth.sr_seed(3, i))
        ev[-1].record()
        torch.cuda.synchronize()
        if r >= 2:
            ub.append(ev[0].elapsed_time(ev[-1]))
    del dW
    # the same block with each layer's dgrad and step in one launch (forge_linear_backward_step_fused);
    # one workspace of counters serves the layers one after another on the stream
    ws = torch.empty(max(forge.backward_workspace_bytes(d["K"]) for d in layers) // 4, dtype=torch.int32,
                     device="cuda")
    ob = []
    ol = [[] for _ in layers]
    for r in range(reps + 2):
        torch.cuda.synchronize()
        ev[0].record()
        for i, d in enumerate(layers):
            forge.linear_backward_step_fused(d["X"], d["dY"], d["W"], d["dX"], d["m"], d["v"], opt="adamw",
                                             hyper=w.hyper, step=2 * reps + 5 + r, seed=synth.sr_seed(3, i),
                                             workspace=ws)
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r >= 2:
            ob.append(ev[0].elapsed_time(ev[-1]))
            for i in range(len(layers)):
                ol[i].append(ev[i].elapsed_time(ev[i + 1]))
    if int(ws[1].item()) != 0:
        raise RuntimeError("the one-launch backward step reported a schedule fault")
    del ws
    # the gradient floor of a framework-style unfused step: every layer's dW is produced by the
    # backward pass and alive until the optimizer runs over all of them (measured as the peak
    # memory above what the fused block holds)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    grads = []
    for i, d in enumerate(layers):
        forge.dgrad(d["dY"], d["W"], d["dX"])
        grads.append(torch.empty((d["N"], d["K"]), dtype=torch.float32, device="cuda"))
        forge.wgrad_gemm(d["X"], d["dY"], grads[-1])
    for i, d in enumerate(layers):
        forge.optimizer_step(grads[i], d["W"], d["m"], d["v"], opt="adamw", hyper=w.hyper, step=2 * reps + 10,
                             seed=synth.sr_seed(3, i))
    torch.cuda.synchronize()
    all_grads_extra = torch.cuda.max_memory_allocated() - base
    del grads
    out["llama8b_block_T8192_dgrad_plus_step"] = {
        "block_us": pctl(block), "tflops_wgrad_plus_dgrad": round(flop / (b50 * 1e-6) / 1e12, 1),
        "per_layer_us_p50": {d["name"]: pctl(per_layer[i])["p50"] for i, d in enumerate(layers)},
        "unfused_block_us": pctl(ub), "unfused_all_gradients_peak_extra_bytes": int(all_grads_extra),
        "fused_peak_extra_bytes": int(fused_extra),
        "one_launch_block_us": pctl(ob),
        "one_launch_per_layer_us_p50": {d["name"]: pctl(ol[i])["p50"] for i, d in enumerate(layers)}}
    del layers
    return out


def _single_fp32(forge, reps, p50_of):
    """The single fp32 linear (W[256, 256], T = 512, fp32 everything, no stochastic rounding):
    fused and unfused."""
    import torch

    import synth
    w = synth.WORKLOADS[1]
    L = w.layers[0]
    X = torch.randn((w.T, L.K), device="cuda") * w.x_std
    dY = torch.randn((w.T, L.N), device="cuda") * w.dy_std
    W = torch.randn((L.N, L.K), device="cuda") * w.w_std
    m, v = torch.zeros_like(W), torch.zeros_like(W)
    dW = torch.empty_like(W)
    # 20 steps back to back between two events, so that the host's per-call time (tens of us
    # of Python marshalling) overlaps the device's instead of adding to it
    fused = p50_of(lambda r: [forge.wgrad_step(X, dY, W, m, v, opt="adamw", hyper=w.hyper, step=20 * r + i + 1, seed=1)
                              for i in range(20)], 10) / 20

    def unf(r):
        for i in range(20):
            forge.wgrad_gemm(X, dY, dW)
            forge.optimizer_step(dW, W, m, v, opt="adamw", hyper=w.hyper, step=1000 + 20 * r + i, seed=1)
    unfused = p50_of(unf, 10) / 20
    flop = 2.0 * w.T * L.N * L.K
    return {"single_fp32_W256x256_T512": {"fused_us": round(fused, 1), "unfused_us": round(unfused, 1),
                                          "tflops": round(flop / (fused * 1e-6) / 1e12, 3)}}


def _qwen_block(forge, reps, randn, p50_of):
    import torch

    import synth
    out = {}
    # Qwen3-14B block, int8 block-64 moments
    w = synth.WORKLOADS[4]
    T = w.T
    layers = []
    for L in w.layers:
        layers.append(dict(name=L.name, N=L.N, K=L.K, X=randn((T, L.K), w.x_std), dY=randn((T, L.N), w.dy_std),
                           W=randn((L.N, L.K), w.w_std),
                           m=torch.zeros((L.N, L.K), dtype=torch.int8, device="cuda"),
                           ms=torch.zeros((L.N * L.K // 64,), device="cuda"),
                           v=torch.zeros((L.N, L.K), dtype=torch.uint8, device="cuda"),
                           vs=torch.zeros((L.N * L.K // 64,), device="cuda")))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)]
    per_layer = [[] for _ in layers]
    block = []
    for r in range(reps + 2):
        torch.cuda.synchronize()
        ev[0].record()
        for i, d in enumerate(layers):
            forge.wgrad_step(d["X"], d["dY"], d["W"], d["m"], d["v"], opt="adamw", hyper=w.hyper, step=r + 1,
                             seed=synth.sr_seed(4, i), m_scale=d["ms"], v_scale=d["vs"])
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r >= 2:
            block.append(ev[0].elapsed_time(ev[-1]))
            for i in range(len(layers)):
                per_layer[i].append(ev[i].elapsed_time(ev[i + 1]))
    flop = sum(2.0 * T * d["N"] * d["K"] for d in layers)
    b50 = pctl(block)["p50"]
    # per layer, the same step with fp32 moments and the contraction alone (fp32 dW), to split
    # the int8 step's time into contraction and epilogue
    dW = torch.empty(max(d["N"] * d["K"] for d in layers), dtype=torch.float32, device="cuda")
    f32_us, gemm_us = {}, {}
    for i, d in enumerate(layers):
        m32 = torch.zeros((d["N"], d["K"]), device="cuda")
        v32 = torch.zeros((d["N"], d["K"]), device="cuda")
        f32_us[d["name"]] = p50_of(lambda r: forge.wgrad_step(d["X"], d["dY"], d["W"], m32, v32, opt="adamw",
                                                              hyper=w.hyper, step=r + 1, seed=synth.sr_seed(4, i)), reps)
        del m32, v32
        gemm_us[d["name"]] = p50_of(lambda r: forge.wgrad_gemm(d["X"], d["dY"], dW[:d["N"] * d["K"]].view(d["N"], d["K"])),
                                    reps)

    # the unfused block, timed like the fused one: the layers one after another, so that each
    # layer's operands and state meet the caches the previous layers left (timing a layer alone,
    # back to back, keeps its 50-200 MB in the 256 MB Infinity Cache and flatters it)
    ub = []
    unf_layer = [[] for _ in layers]
    for r in range(reps + 2):
        torch.cuda.synchronize()
        ev[0].record()
        for i, d in enumerate(layers):
            g = dW[:d["N"] * d["K"]].view(d["N"], d["K"])
            forge.wgrad_gemm(d["X"], d["dY"], g)
            forge.optimizer_step(g, d["W"], d["m"], d["v"], opt="adamw", hyper=w.hyper, step=reps + 3 + r,
                                 seed=synth.sr_seed(4, i), m_scale=d["ms"], v_scale=d["vs"])
            ev[i + 1].record()
        torch.cuda.synchronize()
        if r >= 2:
            ub.append(ev[0].elapsed_time(ev[-1]))
            for i in range(len(layers)):
                unf_layer[i].append(ev[i].elapsed_time(ev[i + 1]))
    del dW
    out["qwen3_14b_block_T4096_int8_states"] = {
        "block_us": pctl(block), "tflops": round(flop / (b50 * 1e-6) / 1e12, 1),
        "per_layer_us_p50": {d["name"]: pctl(per_layer[i])["p50"] for i, d in enumerate(layers)},
        "unfused_block_us": pctl(ub),
        "per_layer_unfused_us_p50": {d["name"]: pctl(unf_layer[i])["p50"] for i, d in enumerate(layers)},
        "per_layer_alone_fp32_states_us_p50": f32_us, "per_layer_alone_contraction_only_us_p50": gemm_us}
    del layers
    return out


def _sweep(forge, reps, randn, fp8, p50_of):
    import torch

    import synth
    out = {}
    # optimizer sweep, W[4096, 4096], T = 16384, bf16 and fp8 inputs
    w = synth.WORKLOADS[5]
    L = w.layers[0]
    T = w.T
    X, dY = randn((T, L.K), w.x_std), randn((T, L.N), w.dy_std)
    X8, xs = fp8(X)
    dY8, ds = fp8(dY)
    sweep = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def sweep_case(fmt, opt):
        W = randn((L.N, L.K), w.w_std)
        m = torch.zeros((L.N, L.K), device="cuda") if "m" in RULE_STATES[opt] else None
        v = torch.zeros((L.N, L.K), device="cuda") if "v" in RULE_STATES[opt] else None
        args = (X, dY, None, None) if fmt == "bf16" else (X8, dY8, xs, ds)
        times = []
        for r in range(reps + 4):
            torch.cuda.synchronize()
            e0.record()
            forge.wgrad_step(args[0], args[1], W, m, v, opt=opt, hyper=w.hyper_for(opt), step=r + 1,
                             seed=synth.sr_seed(5, synth.OPTIMIZERS.index(opt)), x_scale=args[2], dy_scale=args[3])
            e1.record()
            torch.cuda.synchronize()
            if r >= 4:
                times.append(e0.elapsed_time(e1))
        return pctl(times)["p50"]

    cases = [(fmt, opt) for fmt in ("bf16", "fp8") for opt in synth.OPTIMIZERS]
    for fmt, opt in cases:               # one untimed pass over the whole sweep first
        sweep_case(fmt, opt)
    for fmt, opt in cases:
        p50 = sweep_case(fmt, opt)
        sweep[f"{opt}-{fmt}"] = {"us_p50": p50, "tflops": round(2.0 * T * L.N * L.K / (p50 * 1e-6) / 1e12, 1)}
    dW = torch.empty((L.N, L.K), dtype=torch.float32, device="cuda")
    sweep["contraction_only_us_p50"] = {
        "bf16": p50_of(lambda r: forge.wgrad_gemm(X, dY, dW), reps),
        "fp8": p50_of(lambda r: forge.wgrad_gemm(X8, dY8, dW, x_scale=xs, dy_scale=ds), reps)}
    Wu = randn((L.N, L.K), w.w_std)
    mu, vu = torch.zeros((L.N, L.K), device="cuda"), torch.zeros((L.N, L.K), device="cuda")

    def unf(fmt):
        def run(r):
            if fmt == "bf16":
                forge.wgrad_gemm(X, dY, dW)
            else:
                forge.wgrad_gemm(X8, dY8, dW, x_scale=xs, dy_scale=ds)
            forge.optimizer_step(dW, Wu, mu, vu, opt="adamw", hyper=w.hyper_for("adamw"), step=r + 1, seed=3)
        return run
    sweep["unfused_adamw_us_p50"] = {"bf16": p50_of(unf("bf16"), reps), "fp8": p50_of(unf("fp8"), reps)}
    out["sweep_W4096x4096_T16384"] = sweep
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed fused steps run for this long before the warmup steps, so that the GPU's power "
                         "management reaches its steady state (0 disables)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the unfused path, dgrad and the other workloads")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--cpu-steps", type=int, default=6)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cpu-others", action="store_true",
                    help="time the oracle on bounded samples of the other workloads (host only) and print it")
    ap.add_argument("--only", choices=WORKLOAD_PARTS, default=None,
                    help="run only this part of the other workloads (for profiler runs) and print its timings")
    ap.add_argument("--kernel", choices=["fused", "gemm", "optimizer", "dgrad"], default=None,
                    help="run only this kernel of the headline shape (for profiler runs); prints its time")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: runs on one GPU only (--gpus {a.gpus} requested). Across GPUs the fused step shards "
              "W by whole 256x128 tiles with the full token count on each GPU (tensor parallelism), which needs "
              "no exchange on this path, so the per-GPU figure is the one-GPU figure.", file=sys.stderr)
        sys.exit(2)

    if a.cpu_others:
        print(json.dumps(cpu_oracle_other_workloads()), flush=True)
        return

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
    if a.only is not None:
        print(json.dumps(workload_timings(forge, Timer(), 5, parts=(a.only,))), flush=True)
        return

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
    flop = 2.0 * T * N * K

    def tflops_of(ms):
        return flop / (ms * 1e-3) / 1e12

    if a.kernel is not None:
        run_one(a, forge, batches, W, m, v, h, seed, T, N, K)
        return

    t = [0]

    def step(_i):
        t[0] += 1
        Xd, Dd = batches[t[0] % 2]
        forge.wgrad_step(Xd, Dd, W, m, v, opt="adamw", hyper=h, step=t[0], seed=seed)

    timer = Timer()
    # Settle: under sustained load the MI355X's power management first lets a few launches run
    # at a high clock, then throttles below the sustained level and recovers over ~20 launches
    # (per-launch times measured here from a cold start: 608, 670, 756, 863, 847, 808, 771, 737,
    # 709 us ... settling near 610 us).  The timed steps measure the steady state a training run
    # spends its time in; the settle phase's own per-launch times are reported in "extra".
    settle = []
    if a.settle_ms > 0:
        # batches of 8 launches back to back; the host waits only at a batch's end
        ev = [torch.cuda.Event(enable_timing=True)]
        ev[0].record()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < a.settle_ms and len(ev) < 400:
            for _ in range(8):
                step(0)
                ev.append(torch.cuda.Event(enable_timing=True))
                ev[-1].record()
            ev[-9].synchronize()          # keep one batch queued ahead of the host
        torch.cuda.synchronize()
        settle = [round(ev[i].elapsed_time(ev[i + 1]) * 1e3, 1) for i in range(len(ev) - 1)]
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    ms, per_step = timer.warm(step, a.steps)            # the timed region: `steps` fused steps back to back
    fused_peak_extra = torch.cuda.max_memory_allocated() - base_alloc
    tflops = tflops_of(ms)
    # the shader clock over the same back-to-back launches, measured right after the timed region
    clock = clock_during(forge, step, a.steps, 0.6 * a.steps * ms * 1e-3)
    print(f"[bench] fused step {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s, shader clock {clock} MHz", file=sys.stderr,
          flush=True)
    extra = {"fused_us_warm": pctl(per_step), "fused_us_timed": [round(x * 1e3, 1) for x in per_step],
             "settle_launches_us": settle, "fused_peak_extra_bytes": int(fused_peak_extra),
             "shader_clock_mhz_fused": clock}
    if not a.no_extra:
        extra["fused_us_cold"] = pctl(timer.cold(step, 10))
        # unfused two-phase baseline: dW GEMM to HBM, then the optimizer kernel
        torch.cuda.reset_peak_memory_stats()
        base_alloc = torch.cuda.memory_allocated()
        dW = torch.empty((N, K), dtype=torch.float32, device="cuda")

        def gemm(i):
            Xd, Dd = batches[i % 2]
            forge.wgrad_gemm(Xd, Dd, dW)

        def opt_step(_i):
            t[0] += 1
            forge.optimizer_step(dW, W, m, v, opt="adamw", hyper=h, step=t[0], seed=seed)

        def unfused(i):
            gemm(i)
            opt_step(i)
        for i in range(3):
            unfused(i)
        unf_ms, unf_per = timer.warm(unfused, a.steps)
        extra["shader_clock_mhz_unfused"] = clock_during(forge, unfused, a.steps, 0.6 * a.steps * unf_ms * 1e-3)
        unf_peak_extra = torch.cuda.max_memory_allocated() - base_alloc
        gemm_ms, _ = timer.warm(gemm, a.steps)
        opt_ms, _ = timer.warm(opt_step, a.steps)
        unf_cold = timer.cold(unfused, 10)
        # the vendor GEMM (hipBLASLt through torch) for the same product with fp32 out, as context
        try:
            Dt = batches[0][1].t()
            for _ in range(5):
                torch.mm(Dt, batches[0][0], out_dtype=torch.float32)
            vendor_ms, _ = timer.warm(lambda _i: torch.mm(Dt, batches[0][0], out_dtype=torch.float32), a.steps)
            vendor = round(vendor_ms * 1e3, 1)
        except (TypeError, RuntimeError):   # a torch without mm(out_dtype=...)
            vendor = None
        del dW
        # dgrad on the same layer (dX = dY W), bf16 out
        dX = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        dg_ms, _ = timer.warm(lambda _i: forge.dgrad(batches[0][1], W, dX), a.steps)
        del dX
        extra.update({
            "unfused_us": round(unf_ms * 1e3, 1), "unfused_us_warm": pctl(unf_per), "unfused_us_cold": pctl(unf_cold),
            "unfused_gemm_us": round(gemm_ms * 1e3, 1), "unfused_optimizer_us": round(opt_ms * 1e3, 1),
            "fused_speedup_vs_unfused": round(unf_ms / ms, 3), "unfused_peak_extra_bytes": int(unf_peak_extra),
            "vendor_gemm_f32_out_us": vendor, "dgrad_us": round(dg_ms * 1e3, 1),
            "dgrad_tflops": round(tflops_of(dg_ms), 1),
            "optimizer_kernel_hbm_gbs": round(N * K * (4 + 4 + 8 + 8) / (opt_ms * 1e-3) / 1e9, 1),
        })
        print(f"[bench] unfused {gemm_ms * 1e3:.1f} + {opt_ms * 1e3:.1f} us; dgrad {dg_ms * 1e3:.1f} us; "
              f"vendor gemm {vendor} us", file=sys.stderr, flush=True)
        del batches[1]
        torch.cuda.empty_cache()
        print("[bench] timing the other workloads", file=sys.stderr, flush=True)
        extra["workloads"] = workload_timings(forge, timer, 5)

    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic()}
    cpu = None
    if not a.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(a.cpu_rows, a.cpu_steps)
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
