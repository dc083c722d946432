"""Pins of the oracle's storage formats: bf16, stochastic rounding, OCP e4m3, int8 block-64.

Library pins: PyTorch's bfloat16 and float8_e4m3fn conversions.  Closed-form
pins: the exact round-up count of stochastic rounding over all 2^16 random
values, the int8 error bound, exactness of the block maximum.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import numerics


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = numerics.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-40, -1e-41], np.float32),
        # exact ties: low 16 bits == 0x8000
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ]).astype(np.float32)
    ours = numerics.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    q = numerics.bf16_rne(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(numerics.bf16_to_f64(q)))


def _ulp_neighbours(x32):
    """bf16 values just below / above x32 (towards zero / away from zero)."""
    u = x32.view(np.uint32)
    lo = (u >> 16).astype(np.uint16)
    return lo, (lo + 1).astype(np.uint16)


def test_sr_round_up_count_is_exact_fraction():
    """Over all 2^16 random values, x rounds away from zero exactly (u mod 2^16) times."""
    r = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(1)
    for x in rng.standard_normal(40).astype(np.float32):
        u = int(np.array(x, np.float32).view(np.uint32))
        out = numerics.sr_bf16(np.full(1 << 16, x, np.float32), r)
        down, up = _ulp_neighbours(np.array([x], np.float32))
        assert set(np.unique(out).tolist()) <= {int(down[0]), int(up[0])}
        assert int(np.sum(out == up[0])) == (u & 0xFFFF)


def test_sr_unbiased_and_dead_zone():
    """A sub-ULP increment vanishes under round-to-nearest but accumulates under SR."""
    w0 = np.float32(0.02)
    ulp = float(numerics.bf16_to_f64(np.array([(np.array(w0).view(np.uint32) >> 16) + 1], np.uint16))[0]
                - numerics.bf16_to_f64(np.array([np.array(w0).view(np.uint32) >> 16], np.uint16))[0])
    delta = 0.1 * ulp
    n_el, n_steps = 4096, 50
    w_rne = np.full(n_el, numerics.bf16_rne(np.array([w0], np.float32))[0], np.uint16)
    w_sr = w_rne.copy()
    idx = np.arange(n_el, dtype=np.uint64)
    for t in range(1, n_steps + 1):
        w_rne = numerics.bf16_rne((numerics.bf16_to_f64(w_rne) - delta).astype(np.float32))
        x = (numerics.bf16_to_f64(w_sr) - delta).astype(np.float32)
        w_sr = numerics.sr_bf16(x, numerics.sr_bits(3, t, idx))
    start = float(numerics.bf16_to_f64(numerics.bf16_rne(np.array([w0], np.float32)))[0])
    assert np.all(numerics.bf16_to_f64(w_rne) == start)          # frozen in the dead zone
    drift = numerics.bf16_to_f64(w_sr) - start
    want = -n_steps * delta
    # each element's total is a sum of n_steps bounded (1 ULP) unbiased errors
    sd = ulp * np.sqrt(n_steps * 0.25) / np.sqrt(n_el)
    assert abs(drift.mean() - want) < 6 * sd + 1e-3 * abs(want), (drift.mean(), want)


def test_sr_special_values():
    r = np.array([0, 1, 0x7FFF, 0xFFFF], np.uint16)
    for v in (0.0, -0.0, 1.0, -2.5, np.inf, -np.inf):
        out = numerics.sr_bf16(np.full(4, v, np.float32), r)
        exp = numerics.bf16_rne(np.array([v], np.float32))[0]
        assert np.all(out == exp), v
    nan = numerics.sr_bf16(np.array([np.nan, -np.nan, np.array(0x7F800001, np.uint32).view(np.float32)], np.float32),
                           np.array([0xFFFF, 0xFFFF, 0xFFFF], np.uint16))
    assert np.all(np.isnan(numerics.bf16_to_f64(nan)))
    assert nan[1] & 0x8000


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = numerics.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # facts of the format itself
    assert np.nanmax(ours) == 448.0 and ours[0x7E] == 448.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and nan.sum() == 2
    assert ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6 and ours[0x38] == 1.0


@pytest.mark.parametrize("signed", [True, False])
def test_int8_block64_roundtrip_bound(signed):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 512)) * np.exp(rng.standard_normal((8, 512)))
    if not signed:
        x = np.abs(x)
        x[5, 200] = 1e-9                                 # far below half a step of its block
    x[3, 64:128] = 0.0                                   # zero block
    codes, s = numerics.quantize_block64(x, signed)
    assert codes.dtype == (np.int8 if signed else np.uint8)
    assert s.shape == (8, 8)
    # the scale is the block absmax rounded once to fp32
    assert np.array_equal(s, np.abs(x).reshape(8, 8, 64).max(-1).astype(np.float32))
    back = numerics.dequantize_block64(codes, s, signed)
    lv = 127 if signed else 255
    step = np.repeat(s.astype(np.float64), 64, axis=1) / lv
    err = np.abs(back - x)
    if signed:
        assert np.all(err <= 0.5 * step * (1 + 1e-9) + 1e-30)
    else:
        # nearest code within half a step, except that no non-zero value stores code 0: values
        # below half a step store code 1 (one step) instead
        tiny = (x > 0) & (x < 0.5 * step)
        assert tiny.any() and np.all(codes[tiny] == 1)
        assert np.all(err[~tiny] <= 0.5 * step[~tiny] * (1 + 1e-9) + 1e-30)
        assert np.all(codes[x > 0] >= 1) and np.all(codes[x == 0] == 0)
    assert np.all(codes[3, 64:128] == 0) and s[3, 1] == 0
    # the block's largest magnitude maps to the top code and back exactly
    xb = x.reshape(8, 8, 64)
    am = np.argmax(np.abs(xb), axis=2)
    top = np.take_along_axis(codes.reshape(8, 8, 64).astype(np.int64), am[..., None], 2)[..., 0]
    assert np.all((np.abs(top) == lv) | (s == 0))
    # re-quantising the dequantised block is idempotent
    c2, s2 = numerics.quantize_block64(back, signed)
    assert np.array_equal(c2, codes) and np.allclose(s2, s, rtol=1e-6)


@pytest.mark.parametrize("signed", [True, False])
def test_int8_block_with_a_non_finite_value_dequantises_to_nan(signed):
    x = np.abs(np.random.default_rng(3).standard_normal((2, 256))) + 0.1
    x[0, 70] = np.nan                                   # block (0, 1)
    x[1, 200] = np.inf                                  # block (1, 3)
    codes, s = numerics.quantize_block64(x, signed)
    assert np.isnan(s[0, 1]) and np.isnan(s[1, 3])
    assert np.all(codes[0, 64:128] == 0) and np.all(codes[1, 192:256] == 0)
    back = numerics.dequantize_block64(codes, s, signed)
    assert np.all(np.isnan(back[0, 64:128])) and np.all(np.isnan(back[1, 192:256]))
    ok = np.ones((2, 4), bool)
    ok[0, 1] = ok[1, 3] = False
    assert np.all(np.isfinite(s[ok]))
    lv = 127 if signed else 255
    assert np.all(np.abs(back.reshape(2, 4, 64)[ok] - x.reshape(2, 4, 64)[ok]) <= s[ok][:, None] / lv)


def test_int8_second_moment_floor_keeps_adamw_bounded():
    """Why no non-zero second moment stores code 0 (FORGE explainer, Technical Summary section 3:
    full-precision fidelity with int8 states).  Two AdamW steps at the Qwen3-14B workload's
    gradient scale with the moments stored in block-64 int8 after step 1: with the floor every
    update stays within a few learning rates (the fp32 bound is about lr (1 - b1) / sqrt(1 - b2)),
    while plain nearest rounding, which stores about 1 value in 11 as 0, lets updates grow by
    two orders of magnitude."""
    from oracle import optimizers
    rng = np.random.default_rng(14)
    rows, cols = 64, 4096
    h = synth.default_hyper("adamw")
    W0 = rng.standard_normal((rows, cols)) * 0.02
    g1 = rng.standard_normal((rows, cols)) * 0.064      # |g| of X ~ N(0,1), dY ~ N(0,1e-3), T = 4096
    g2 = rng.standard_normal((rows, cols)) * 0.064
    z = np.zeros((rows, cols))
    W1, m1, v1 = optimizers.update("adamw", h, 1, g1, W0, z, z)

    def second_step(vq):
        mq = numerics.dequantize_block64(*numerics.quantize_block64(m1, True), True)
        W2, _, _ = optimizers.update("adamw", h, 2, g2, W1, mq, vq)
        return np.abs(W2 - W1 * (1 - 1e-3 * 0.01)) / 1e-3   # update size in learning rates

    with_floor = second_step(numerics.dequantize_block64(*numerics.quantize_block64(v1, False), False))
    xb = v1.reshape(rows, cols // 64, 64)
    sc = xb.max(-1, keepdims=True).astype(np.float32).astype(np.float64)
    plain = second_step((np.rint(xb * 255 / sc) * sc / 255).reshape(rows, cols))
    ref = second_step(v1)
    assert float(np.mean(np.rint(xb * 255 / sc) == 0)) > 0.05
    assert with_floor.max() < 4.0 and ref.max() < 4.0
    assert plain.max() > 50.0


def test_int8_blocks_are_64_consecutive_row_elements():
    x = np.full((2, 256), 1e-3)
    x[0, 70] = 5.0                                     # lives in block (0, 1): cols 64..127
    codes, s = numerics.quantize_block64(x, True)
    assert s[0, 1] == np.float32(5.0)
    assert np.all(s[0, [0, 2, 3]] == np.float32(1e-3)) and np.all(s[1] == np.float32(1e-3))
    assert np.all(codes[0, 64:128][np.arange(64) != 6] == 0)   # 1e-3 * 127 / 5 rounds to 0
    assert np.all(codes[0, :64] == 127)


def test_block64_quantisation_beats_block2048():
    """FORGE explainer, Technical Summary section 2 "Precision and Fidelity": int8 moments use
    blocks of 64 instead of the 2048 of common 8-bit optimizers to reduce quantisation error.
    Moments after a few AdamW steps on heavy-tailed gradients (a few large entries per row, as
    real gradients have) lose less to block-64 absmax quantisation than to block-2048."""
    from oracle import optimizers
    rng = np.random.default_rng(5)
    rows, cols = 64, 4096
    h = synth.default_hyper("adamw")
    m = np.zeros((rows, cols))
    v = np.zeros((rows, cols))
    W = rng.standard_normal((rows, cols)) * 0.02
    for t in range(1, 6):
        g = rng.standard_t(3, size=(rows, cols)) * 1e-3
        W, m, v = optimizers.update("adamw", h, t, g, W, m, v)

    def err(x, block, signed):
        xb = x.reshape(rows, cols // block, block)
        s = np.abs(xb).max(-1, keepdims=True)
        lv = 127 if signed else 255
        q = np.rint(np.where(s > 0, xb / np.where(s > 0, s, 1) * lv, 0))
        return float(np.sqrt(np.mean((q * s / lv - xb) ** 2)))
    for x, signed in ((m, True), (v, False)):
        e64, e2048 = err(x, 64, signed), err(x, 2048, signed)
        assert e64 < 0.7 * e2048, (e64, e2048)
    # and the oracle's own block-64 quantiser has the block-64 error
    codes, scales = numerics.quantize_block64(m, True)
    deq = numerics.dequantize_block64(codes, scales, True)
    assert abs(float(np.sqrt(np.mean((deq - m) ** 2))) - err(m, 64, True)) < 1e-3 * err(m, 64, True) + 1e-12


@pytest.mark.parametrize("signed", [True, False])
def test_blocks_of_any_size_with_a_ragged_last_block(signed):
    """Blocks of 2048 on rows of 5120 elements (the Qwen3-14B hidden size): two full blocks and
    one of 1024.  Each block's scale is its own absmax; the error stays within half a step of
    its block (or one step for the second-moment floor)."""
    from oracle import dynmap
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 5120)) * 1e-3
    if not signed:
        x = np.abs(x)
    codes, s = numerics.quantize_blocks(x, signed, 2048)
    assert s.shape == (3, 3)
    for b, (c0, c1) in enumerate(((0, 2048), (2048, 4096), (4096, 5120))):
        assert np.array_equal(s[:, b], np.abs(x[:, c0:c1]).max(1).astype(np.float32))
    back = numerics.dequantize_blocks(codes, s, signed, 2048)
    step = np.repeat(s.astype(np.float64), 2048, axis=1)[:, :5120] / (127 if signed else 255)
    assert np.all(np.abs(back - x) <= step * (1 + 1e-9))
    dc, ds = dynmap.quantize_blocks(x, signed, 2048)
    assert np.array_equal(ds, s)
    # dynamic map: within half a step of the value's decade (10^-(E+1), 10^-E] of the block scale
    sc = np.repeat(ds.astype(np.float64), 2048, axis=1)[:, :5120]
    B = 7 if signed else 8
    y = np.abs(x) / sc
    E = np.clip(np.ceil(-np.log10(np.maximum(y, 1e-30))) - 1, 0, B - 1)
    half = 0.5 * 0.9 * 10.0 ** (-E) / 2.0 ** (B - 1 - E) * sc
    err = np.abs(dynmap.dequantize_blocks(dc, ds, signed, 2048) - x)
    assert np.all(err <= half * (1 + 1e-9) + 10.0 ** (-(B - 1)) * sc)
