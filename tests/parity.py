"""Helpers of the GPU parity tests: moving seeded inputs to the device, running the library,
and comparing its outputs with the CPU oracle.

Acceptance (tolerances from the workload specification):
  * fp32 moments and the fp32 weight before rounding: |gpu - ref| <= 1e-6 + 1e-4 |ref|,
    with moments additionally held to a tensor-relative floor (|gpu - ref| <= 1e-4 |ref| +
    1e-7 max|ref|), because 1e-6 absolute is larger than a second moment itself;
  * bf16 weights: within 1 bf16 ULP;
  * int8 moments: codes within 1, block scales within rel 1e-4.

Where several results are correct they are all accepted, and only what is unique is
compared:
  * the gradient of the kernel is a fp32 sum whose order differs from the oracle's; the
    explainer pages (FORGE, gist.science, Technical Summary section 2 "Precision and
    Fidelity") name the summation order as the only deviation.  Any fp32 sum of T products
    differs from the exact one by at most tau = 2 (T + 1) 2^-24 sum_t |dY[t,n] X[t,k]|
    (first-order bound for any order, doubled for safety).  The weight of an element is
    accepted if it lies within the tolerance of the range the oracle's rule gives over
    gradients in [g - tau, g + tau] ("envelope");
  * inputs on a dyadic grid make every fp32 partial sum exact (tau = 0), so those cases
    are compared without any envelope;
  * Lion's sign(c) is ambiguous where |c| is within fp32 rounding of 0.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import dynmap, numerics, optimizers, wgrad

U32 = 2.0 ** -24


# ----------------------------------------------------------------------------- device transfer
def dev_operand(op: synth.Operand):
    """synth.Operand -> (device tensor, device scale or None)."""
    if op.fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(op.data)).cuda(), None
    if op.fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(op.data).view(np.int16)).cuda().view(torch.bfloat16), None
    if op.fmt == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(op.data)).cuda().view(torch.float8_e4m3fn)
        return t, torch.tensor([float(op.scale)], dtype=torch.float32, device="cuda")
    raise ValueError(op.fmt)


def dev_weight(W: np.ndarray, w_fmt: str):
    if w_fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).cuda().view(torch.bfloat16)


def host_weight(t, w_fmt: str) -> np.ndarray:
    if w_fmt == "f32":
        return t.cpu().numpy().copy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()


def dev_state(st, state_fmt: str, signed: bool):
    """oracle state (float32 array or (codes, scales)) -> (device tensor, device scales or None)."""
    if st is None:
        return None, None
    if state_fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(st, np.float32)).cuda(), None
    codes, scales = st
    c = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    return c, torch.from_numpy(np.ascontiguousarray(scales.reshape(-1), np.float32)).cuda()


def host_state(t, s, state_fmt: str):
    if t is None:
        return None
    if state_fmt == "f32":
        return t.cpu().numpy().copy()
    codes = t.cpu().numpy().copy()
    return codes, s.cpu().numpy().reshape(codes.shape[0], codes.shape[1] // 64).copy()


class DeviceStep:
    """Device copies of W, m, v for one layer, stepped by the library."""

    def __init__(self, W, m, v, w_fmt, state_fmt):
        self.w_fmt, self.state_fmt = w_fmt, state_fmt
        self.W = dev_weight(W, w_fmt)
        self.m, self.ms = dev_state(m, state_fmt, True)
        self.v, self.vs = dev_state(v, state_fmt, False)

    @property
    def state_map(self):
        return "dynamic" if self.state_fmt == "int8dyn" else "linear"

    def fused(self, lib, X: synth.Operand, dY: synth.Operand, opt, hyper, step, seed, preround=False, sr=True):
        Xd, xs = dev_operand(X)
        Dd, ds = dev_operand(dY)
        pre = torch.empty(self.W.shape, dtype=torch.float32, device="cuda") if preround else None
        lib.wgrad_step(Xd, Dd, self.W, self.m, self.v, opt=opt, hyper=hyper, step=step, seed=seed,
                       x_scale=xs, dy_scale=ds, m_scale=self.ms, v_scale=self.vs, w_preround_out=pre, sr=sr,
                       state_map=self.state_map)
        return pre

    def unfused(self, lib, X, dY, opt, hyper, step, seed, preround=False, sr=True):
        Xd, xs = dev_operand(X)
        Dd, ds = dev_operand(dY)
        dW = torch.empty(self.W.shape, dtype=torch.float32, device="cuda")
        lib.wgrad_gemm(Xd, Dd, dW, x_scale=xs, dy_scale=ds)
        pre = torch.empty(self.W.shape, dtype=torch.float32, device="cuda") if preround else None
        lib.optimizer_step(dW, self.W, self.m, self.v, opt=opt, hyper=hyper, step=step, seed=seed,
                           m_scale=self.ms, v_scale=self.vs, w_preround_out=pre, sr=sr, state_map=self.state_map)
        return pre, dW

    def host(self):
        torch.cuda.synchronize()
        return (host_weight(self.W, self.w_fmt), host_state(self.m, self.ms, self.state_fmt),
                host_state(self.v, self.vs, self.state_fmt))


# ----------------------------------------------------------------------------- error bounds
def grad_bound(X: synth.Operand, dY: synth.Operand) -> np.ndarray:
    """tau: bound on |fp32 sum - exact| for any summation order of the T products."""
    X64, dY64 = wgrad.decode_operand(X), wgrad.decode_operand(dY)
    T = X64.shape[0]
    s = wgrad.wgrad_abs(X64, dY64)
    tau = 2.0 * (T + 1) * U32 * s
    if X.fmt == "fp8":  # two more fp32 roundings: scale product and the scaling of the sum
        tau = tau + 4.0 * U32 * np.abs(wgrad.wgrad(X64, dY64))
    return tau


# ----------------------------------------------------------------------------- comparisons
def bf16_ulp(bits: np.ndarray) -> np.ndarray:
    """Size of one bf16 ULP at each value."""
    x = numerics.bf16_to_f64(bits)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance between bf16 bit patterns counted in representable steps (sign aware)."""
    def key(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def moment_close(gpu: np.ndarray, ref64: np.ndarray, what: str, lo=None, hi=None):
    """fp32 moment vs the oracle; [lo, hi] is the range of correct values (default: the oracle's)."""
    gpu = gpu.astype(np.float64)
    lo = ref64 if lo is None else lo
    hi = ref64 if hi is None else hi
    scale = float(np.max(np.abs(ref64))) if ref64.size else 0.0
    tol = 1e-4 * np.maximum(np.abs(lo), np.abs(hi)) + min(1e-6, 1e-7 * scale)
    bad = (gpu < lo - tol) | (gpu > hi + tol)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements off; first: got {gpu.flat[i]:.9e}, "
                             f"want [{lo.flat[i]:.9e}, {hi.flat[i]:.9e}]")


def code_rank(codes: np.ndarray, state_fmt: str) -> np.ndarray:
    """Position of 8-bit codes in value order: the code itself for the linear map (int8 signed,
    uint8 unsigned); sign and magnitude pattern for the dynamic map, whose magnitudes increase
    with the 7 (signed) or 8 (unsigned) magnitude bits."""
    c = np.asarray(codes)
    if state_fmt == "int8dyn" and c.dtype == np.int8:
        u = c.view(np.uint8).astype(np.int64)
        return np.where(u & 0x80, -(u & 0x7F), u & 0x7F)
    return c.astype(np.int64)


def int8_state_close(gpu, ref, what: str, state_fmt: str = "int8"):
    (gc, gs), (rc, rs) = gpu, ref
    d = np.abs(code_rank(gc, state_fmt) - code_rank(rc, state_fmt))
    assert d.max(initial=0) <= 1, f"{what}: 8-bit codes differ by {int(d.max())} steps"
    np.testing.assert_allclose(gs, rs, rtol=1e-4, atol=0, err_msg=f"{what} block scales")


def state_close(gpu, ref_stored, ref64, state_fmt, what, lo=None, hi=None):
    if gpu is None:
        assert ref_stored is None
        return
    if state_fmt == "f32":
        moment_close(gpu, ref64, what, lo, hi)
    else:
        int8_state_close(gpu, ref_stored, what, state_fmt)


def arith_slack(W_old, w_fmt, W_new64) -> np.ndarray:
    """Bound on the fp32 rounding of the rule's own arithmetic for the new weight.

    The kernel forms decay * W and the update with a handful of fp32 operations (each
    within one rounding, sqrt and reciprocal within 1 ulp); 16 roundings of the larger of
    the old and new magnitudes bound it.  It matters only where the new weight is the
    small difference of two larger numbers.
    """
    W64 = numerics.bf16_to_f64(W_old) if w_fmt == "bf16" else np.asarray(W_old, np.float32).astype(np.float64)
    return 16 * U32 * (np.abs(W64) + np.abs(W_new64))


def weight_close(gpu_W: np.ndarray, ref: dict, w_fmt: str, lo=None, hi=None, what="W", slack=0.0):
    """gpu weight vs the oracle's; [lo, hi] (float64) is the range of correct pre-rounding values."""
    if lo is None:
        lo = hi = ref["W64"]
    if w_fmt == "f32":
        x = gpu_W.astype(np.float64)
        tol = 1e-6 + 1e-4 * np.maximum(np.abs(lo), np.abs(hi))
        bad = (x < lo - tol) | (x > hi + tol)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements outside tolerance"
        return
    x = numerics.bf16_to_f64(gpu_W)
    u = np.maximum(bf16_ulp(numerics.bf16_rne(lo.astype(np.float32))), bf16_ulp(numerics.bf16_rne(hi.astype(np.float32))))
    u = u * (1 + 1e-6) + slack
    bad = (x < lo - u) | (x > hi + u)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} bf16 elements more than 1 ULP outside "
                             f"[{lo.flat[i]:.8e}, {hi.flat[i]:.8e}] (got {x.flat[i]:.8e})")


def preround_close(gpu_pre: np.ndarray, lo, hi, what="W before rounding"):
    x = gpu_pre.astype(np.float64)
    tol = 1e-6 + 1e-4 * np.maximum(np.abs(lo), np.abs(hi))
    bad = (x < lo - tol) | (x > hi + tol)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside tolerance; first: got {x.flat[i]:.9e}, "
                             f"want [{np.asarray(lo).flat[i]:.9e}, {np.asarray(hi).flat[i]:.9e}]")


def _adam_critical_points(opt, hyper, t, m64, v64):
    """Interior extrema of the Adam family's step as a function of the effective gradient x.

    Each rule's step has the form (A + B x) / (sqrt(C + D x^2) + E) (times a positive
    constant): AdamW and NAdam with v divided by its bias correction, RAdam's rectified branch
    with v as it is (its other branch is linear in x).  Setting the derivative to zero gives
    B E S = A D x - B C with S = sqrt(C + D x^2); squared, the quadratic
    (A^2 D^2 - B^2 E^2 D) x^2 - 2 A B C D x + B^2 C (C - E^2) = 0, whose real roots hold every
    critical point (they are only candidates: the envelope takes the oracle's value there)."""
    p = optimizers.hyper64(hyper)
    s = optimizers.step_scalars(opt, hyper, t)
    b1, b2, eps = p["beta1"], p["beta2"], p["eps"]
    if opt == "radam" and not s["rectified"]:
        return []
    A, B = b1 * m64, np.full_like(m64, 1.0 - b1)
    if opt == "nadam":
        c_g = p["lr"] * (1.0 - s["mu"]) / (1.0 - s["prod"])
        c_m = p["lr"] * s["mu_next"] / (1.0 - s["prod_next"])
        A, B = c_m * b1 * m64, np.full_like(m64, c_g + c_m * (1.0 - b1))
    if opt == "radam":
        C, D = b2 * v64, 1.0 - b2
    else:
        C, D = b2 * v64 / s["bc2"], (1.0 - b2) / s["bc2"]
    E = eps
    qa = A * A * D * D - B * B * E * E * D
    qb = -2.0 * A * B * C * D
    qc = B * B * C * (C - E * E)
    out = []
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        disc = qb * qb - 4.0 * qa * qc
        sq = np.sqrt(np.maximum(disc, 0.0))
        q = -0.5 * (qb + np.where(qb >= 0, sq, -sq))
        for r in (q / qa, qc / q, -qc / qb):          # the last one: the root when qa == 0
            out.append(np.where(np.isfinite(r) & (disc >= 0), r, np.nan))
    return out


def _zoom_extremes(fn, g, tau, lo_v, hi_v, n=129, k=17, rounds=10, chunk=1 << 16):
    """Per element, the minimum and maximum of fn(g', sel) over g' in [g - tau, g + tau], folded
    into lo_v / hi_v.  fn maps gradients of the elements `sel` (flat indices) to their values.

    A grid of n points, then `rounds` zooms around the best point: each zoom samples k points
    over one cell either side of it and shrinks the cell by (k - 1) / 2.  Where the function
    has one extremum near the best grid point, that point is next to it, so the zoom window
    holds it; the final cell is 2 tau / (n - 1) / 8^rounds wide.  Elements go in chunks.
    """
    gf, tf = g.ravel(), tau.ravel()
    lo_f, hi_f = np.array(lo_v, np.float64).ravel(), np.array(hi_v, np.float64).ravel()
    F = np.linspace(-1.0, 1.0, n)
    S = np.linspace(-1.0, 1.0, k)
    for c0 in range(0, gf.size, chunk):
        sel = np.arange(c0, min(gf.size, c0 + chunk))
        gc, tc = gf[sel], tf[sel]
        idx = np.arange(sel.size)
        Xg = gc[None, :] + tc[None, :] * F[:, None]
        Vg = np.stack([fn(x, sel) for x in Xg])
        for pick, better in ((np.argmin, np.less), (np.argmax, np.greater)):
            j = pick(Vg, axis=0)
            bx, bv = Xg[j, idx], Vg[j, idx]
            half = 2.0 * tc / (n - 1)
            for _ in range(rounds):
                Xs = np.clip(bx[None, :] + half[None, :] * S[:, None], gc - tc, gc + tc)
                Vs = np.stack([fn(x, sel) for x in Xs])
                jj = pick(Vs, axis=0)
                cx, cv = Xs[jj, idx], Vs[jj, idx]
                b = better(cv, bv)
                bx, bv = np.where(b, cx, bx), np.where(b, cv, bv)
                half = half * 2.0 / (k - 1)
            if pick is np.argmin:
                lo_f[sel] = np.minimum(lo_f[sel], bv)
            else:
                hi_f[sel] = np.maximum(hi_f[sel], bv)
    return lo_f.reshape(g.shape), hi_f.reshape(g.shape)


def envelope(opt, hyper, t, g, tau, W_old, m_old, v_old, w_fmt, state_fmt, dense=False):
    """Range of the oracle's new fp64 weight (and moments) over gradients g' in [g - tau, g + tau].

    Returns (lo, hi, {"m": (lo, hi), "v": (lo, hi)}) for the moments the rule keeps.  The
    range is the oracle's value at the ends, the midpoints and g itself, and where they lie in
    the interval, at the point where the effective gradient (g' plus any coupled L2 term) is
    zero (the minimum of v) and, for the Adam family, at the critical points of its step (the
    interior extrema of the new weight when the moments are non-zero).  The other moments and
    rules are monotone in the effective gradient.  dense=True also runs a grid-and-zoom search
    for the weight's extremes (a check on the candidates above, for few elements).
    """
    W64 = numerics.bf16_to_f64(W_old) if w_fmt == "bf16" else np.asarray(W_old, np.float32).astype(np.float64)
    m64 = wgrad.decode_state(m_old, state_fmt, True)
    v64 = wgrad.decode_state(v_old, state_fmt, False)
    g = np.asarray(g, np.float64)
    tau = np.broadcast_to(np.asarray(tau, np.float64), g.shape)
    p = optimizers.hyper64(hyper)
    l2 = 0.0 if optimizers.decoupled(opt, p["wd_mode"]) else p["wd"]
    pts = [g - tau, g - 0.5 * tau, g, g + 0.5 * tau, g + tau]
    res = [optimizers.update(opt, hyper, t, gp, W64, m64, v64) for gp in pts]
    # interior candidates, as effective gradients x (g' = x - l2 W); those outside the range
    # take the value at g instead
    cands = [np.zeros_like(g)]
    if opt in ("adamw", "nadam", "radam") and m64 is not None and v64 is not None:
        cands += _adam_critical_points(opt, hyper, t, np.broadcast_to(m64, g.shape), np.broadcast_to(v64, g.shape))
    for x in cands:
        gp = x - l2 * W64
        inside = np.isfinite(gp) & (g - tau <= gp) & (g + tau >= gp)
        if inside.any():
            z = optimizers.update(opt, hyper, t, np.where(inside, gp, g), W64, m64, v64)
            res.append(tuple(None if a is None else np.where(inside, a, b) for a, b in zip(z, res[2])))
    outs = [r[0] for r in res]
    lo = np.minimum.reduce(outs)
    hi = np.maximum.reduce(outs)
    if dense and g.size:
        flat = lambda a, sel: None if a is None else np.broadcast_to(a, g.shape).ravel()[sel]
        lo, hi = _zoom_extremes(lambda x, sel: optimizers.update(opt, hyper, t, x, flat(W64, sel), flat(m64, sel),
                                                                 flat(v64, sel))[0], g, tau, lo, hi)
    mom = {}
    for j, name in ((1, "m"), (2, "v")):
        if res[0][j] is not None:
            vals = [r[j] for r in res]
            mom[name] = (np.minimum.reduce(vals), np.maximum.reduce(vals))
    if opt == "lion":
        # sign(c) with c = b1 m + (1 - b1) g is ambiguous where c is within fp32 rounding of 0
        p = optimizers.hyper64(hyper)
        c = p["beta1"] * m64 + (1 - p["beta1"]) * g
        amb = np.abs(c) <= 4 * U32 * (np.abs(p["beta1"] * m64) + np.abs((1 - p["beta1"]) * g)) + (1 - p["beta1"]) * tau
        if amb.any():
            Wd = W64 * (1 - p["lr"] * p["wd"]) if optimizers.decoupled("lion", p["wd_mode"]) else W64
            lo = np.where(amb, np.minimum(lo, Wd - p["lr"]), lo)
            hi = np.where(amb, np.maximum(hi, Wd + p["lr"]), hi)
    return lo, hi, mom


def moment_tol(lo, hi) -> np.ndarray:
    """The fp32-moment tolerance of moment_close, for the range [lo, hi]."""
    scale = float(np.max(np.maximum(np.abs(lo), np.abs(hi)))) if np.size(lo) else 0.0
    return 1e-4 * np.maximum(np.abs(lo), np.abs(hi)) + min(1e-6, 1e-7 * scale)


def int8_envelope_close(gpu, lo, hi, signed: bool, what: str):
    """int8 block-64 moment against the range [lo, hi] (float64) of correct new values.

    The block scale must lie within rel 1e-4 of the block's absmax for some choice of values
    in the range; each code within one step of the range quantised with the device's own
    scale (code = rint(x * levels / scale)).  With lo == hi this is the plain rule: codes
    within 1, scales within rel 1e-4.
    """
    codes, scales = gpu
    rows, cols = codes.shape
    lv = numerics.levels(signed)
    tol = moment_tol(lo, hi)
    lo_, hi_ = lo - tol, hi + tol
    a_hi = np.maximum(np.abs(lo_), np.abs(hi_))
    a_lo = np.where((lo_ <= 0) & (hi_ >= 0), 0.0, np.minimum(np.abs(lo_), np.abs(hi_)))
    s_hi = a_hi.reshape(rows, -1, numerics.BLOCK).max(-1)
    s_lo = a_lo.reshape(rows, -1, numerics.BLOCK).max(-1)
    sc = scales.astype(np.float64)
    bad = (sc < s_lo * (1 - 1e-4)) | (sc > s_hi * (1 + 1e-4))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} block scales off; first: got {sc.flat[i]:.9e}, "
                             f"want [{s_lo.flat[i]:.9e}, {s_hi.flat[i]:.9e}]")
    s = np.repeat(sc, numerics.BLOCK, axis=1)
    pos = s > 0
    safe = np.where(pos, s, 1.0)
    qlo = np.where(pos, lo_ * lv / safe, 0.0)
    qhi = np.where(pos, hi_ * lv / safe, 0.0)
    c = codes.astype(np.float64)
    bad = (c < qlo - 1.5) | (c > qhi + 1.5) | (~pos & (c != 0))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} int8 codes off; first: got {int(c.flat[i])}, "
                             f"want [{qlo.flat[i]:.3f}, {qhi.flat[i]:.3f}] +- 1")


def init_states(opt, state_fmt, rng, N, K):
    """Non-trivial previous moments in the rule's domain (v >= 0)."""
    m, v = wgrad.init_states(opt, N, K, state_fmt)
    mm = rng.standard_normal((N, K)) * 2e-3
    vv = np.abs(rng.standard_normal((N, K))) * 1e-5
    if opt == "adagrad":
        vv = vv * 10
    if state_fmt == "f32":
        m = None if m is None else mm.astype(np.float32)
        v = None if v is None else vv.astype(np.float32)
    else:
        q = dynmap if state_fmt == "int8dyn" else numerics
        m = None if m is None else q.quantize_block64(mm, True)
        v = None if v is None else q.quantize_block64(vv, False)
    return m, v


def compare(ref, got_W, got_m, got_v, pre, w_fmt, state_fmt, W_old, env=None, tag="", lion=None):
    """env = (lo, hi, moment ranges) from parity.envelope for inputs whose sums are not exact.

    lion = (hyper, step, m_old, v_old) for Lion with exact sums: sign(c) of c = b1 m + (1 - b1) g
    is still ambiguous where c is within fp32 rounding of 0, so the range with tau = 0 is used.
    """
    if env is None and lion is not None:
        h, t, m_old, v_old = lion
        env = envelope("lion", h, t, ref["g"], np.zeros_like(ref["g"]), W_old, m_old, v_old, w_fmt, state_fmt)
    lo, hi, mom = env if env is not None else (None, None, {})
    slack = arith_slack(W_old, w_fmt, ref["W64"])
    weight_close(got_W, ref, w_fmt, lo, hi, what=f"{tag} W", slack=slack)
    if pre is not None:
        preround_close(pre, ref["W64"] if lo is None else lo, ref["W64"] if hi is None else hi, what=f"{tag} W32")
    state_close(got_m, ref["m"], ref["m64"], state_fmt, f"{tag} m", *mom.get("m", (None, None)))
    state_close(got_v, ref["v"], ref["v64"], state_fmt, f"{tag} v", *mom.get("v", (None, None)))


def norm_gate(gpu: np.ndarray, ref64: np.ndarray, what: str, tol: float = 1e-5) -> float:
    """Tensor-wide gate: ||gpu - ref|| / ||ref|| <= tol (returns the ratio)."""
    g = np.asarray(gpu, np.float64)
    num = float(np.linalg.norm((g - ref64).ravel()))
    den = float(np.linalg.norm(np.asarray(ref64, np.float64).ravel()))
    r = num / den if den > 0 else num
    assert r <= tol, f"{what}: ||gpu - ref|| / ||ref|| = {r:.3e} > {tol:.0e}"
    return r


def grad_bound_rows(X64: np.ndarray, dY64_rows: np.ndarray, g: np.ndarray, fp8: bool) -> np.ndarray:
    """grad_bound for the rows of W whose dY columns are given (decoded inputs)."""
    T = X64.shape[0]
    tau = 2.0 * (T + 1) * U32 * (np.abs(dY64_rows).T @ np.abs(X64))
    if fp8:
        tau = tau + 4.0 * U32 * np.abs(g)
    return tau


def dx_close(got_bits: np.ndarray, dY64: np.ndarray, W64: np.ndarray, what: str = "dX"):
    """bf16 dX (bits) against the exact dY W: within the bound on any fp32 summation order of the
    N products, tau = 2 (N + 1) 2^-24 sum_n |dY W|, plus one bf16 ULP of the rounding."""
    ref = dY64 @ W64
    tau = 2.0 * (dY64.shape[1] + 1) * U32 * (np.abs(dY64) @ np.abs(W64))
    got = numerics.bf16_to_f64(got_bits)
    u = bf16_ulp(numerics.bf16_rne(ref.astype(np.float32))) * (1 + 1e-6)
    bad = np.abs(got - ref) > tau + u
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements beyond 1 ULP + sum bound; first: "
                             f"got {got.flat[i]:.8e}, exact {ref.flat[i]:.8e}, bound {tau.flat[i] + u.flat[i]:.3e}")
