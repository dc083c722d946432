"""Pins of the oracle's dynamic 8-bit moment map (oracle/dynmap.py).

The map is written from the published description of dynamic tree quantisation: a sign bit, a
run of E zero bits (decimal exponent), an indicator bit, F fraction bits.  Pinned here:
  * the bit layout itself, decoded independently of the oracle's table builder;
  * encoding is the nearest table value, checked by brute force over the whole table;
  * every code round-trips; the error within a decade is at most half a step;
  * the block codec's special cases (block maximum exact, zero block, non-finite block, no
    non-zero second moment stored as 0);
  * the property the description gives for the map: on values spread over several decades its
    relative error is far below the linear absmax code's.
"""
import numpy as np
import pytest

from oracle import dynmap, numerics


@pytest.mark.parametrize("signed", [True, False])
def test_bit_layout(signed):
    B = 7 if signed else 8
    mags = dynmap.code_magnitudes(signed)
    assert mags[0] == 0.0
    for p in range(1, 1 << B):
        bits = format(p, f"0{B}b")
        E = bits.index("1")                       # the zero run before the indicator bit
        frac = bits[E + 1:]
        F = len(frac)
        f = int(frac, 2) if frac else 0
        lo, hi = 10.0 ** (-E - 1), 10.0 ** (-E)
        want = lo + (hi - lo) * (f + 1) / 2 ** F    # decade (10^-(E+1), 10^-E] in 2^F equal steps
        assert mags[p] == pytest.approx(want, rel=1e-15), (p, bits)
    assert mags.max() == 1.0 and np.sort(mags)[1] == pytest.approx(1e-6 if signed else 1e-7)
    assert len(np.unique(mags)) == 1 << B          # all distinct (0 once)


@pytest.mark.parametrize("signed", [True, False])
def test_encode_is_nearest_by_brute_force(signed):
    rng = np.random.default_rng(7)
    y = np.concatenate([10.0 ** rng.uniform(-9, 0, 20000), rng.uniform(0, 1, 5000), [0.0, 1.0]])
    if signed:
        y = y * np.where(rng.random(y.size) < 0.5, -1.0, 1.0)
    got = dynmap.decode_codes(dynmap.encode_relative(y, signed), signed)
    table = dynmap.code_magnitudes(signed)
    vals = np.concatenate([table, -table[1:]]) if signed else table
    best = np.min(np.abs(vals[None, :] - y[:, None]), axis=1)
    err = np.abs(got - y)
    if signed:
        assert np.all(err <= best * (1 + 1e-12) + 1e-300)
    else:
        small = (y > 0) & (y < 0.5e-7)                # the floor: non-zero takes the smallest code
        assert np.all(got[small] == pytest.approx(1e-7))
        assert np.all(err[~small] <= best[~small] * (1 + 1e-12) + 1e-300)


@pytest.mark.parametrize("signed", [True, False])
def test_every_code_round_trips(signed):
    codes = np.arange(256, dtype=np.uint8)
    if signed:
        codes = codes[codes != 0x80].view(np.int8)     # negative zero decodes to 0
    back = dynmap.encode_relative(dynmap.decode_codes(codes, signed), signed)
    assert np.array_equal(back.view(np.uint8), codes.view(np.uint8))


@pytest.mark.parametrize("signed", [True, False])
def test_error_within_a_decade_is_half_a_step(signed):
    B = 7 if signed else 8
    rng = np.random.default_rng(8)
    y = 10.0 ** rng.uniform(-(B - 1), 0, 50000)
    got = dynmap.decode_codes(dynmap.encode_relative(y, signed), signed)
    E = np.clip(np.ceil(-np.log10(y)) - 1, 0, B - 1)   # decade (10^-(E+1), 10^-E]
    step = 0.9 * 10.0 ** (-E) / 2.0 ** (B - 1 - E)
    assert np.all(np.abs(got - y) <= 0.5 * step * (1 + 1e-9))


@pytest.mark.parametrize("signed", [True, False])
def test_block_codec_special_cases(signed):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 256)) * 1e-3
    if not signed:
        x = np.abs(x)
        x[1, 5] = 1e-15                                 # far below the smallest code
    x[2, 64:128] = 0.0
    x[3, 200] = np.nan
    codes, s = dynmap.quantize_block64(x, signed)
    assert codes.dtype == (np.int8 if signed else np.uint8)
    assert np.array_equal(s[:3], np.abs(x[:3]).reshape(3, 4, 64).max(-1).astype(np.float32))
    back = dynmap.dequantize_block64(codes, s, signed)
    # the block maximum maps to the top code and back exactly
    xb, bb = x[:2].reshape(2, 4, 64), back[:2].reshape(2, 4, 64)
    am = np.argmax(np.abs(xb), axis=2)
    assert np.array_equal(np.take_along_axis(bb, am[..., None], 2), np.take_along_axis(xb, am[..., None], 2).astype(np.float32).astype(np.float64))
    assert s[2, 1] == 0 and np.all(codes[2, 64:128] == 0)
    assert np.isnan(s[3, 3]) and np.all(codes[3, 192:256] == 0) and np.all(np.isnan(back[3, 192:256]))
    if not signed:
        assert np.all(codes[:2][x[:2] > 0] != 0)


def test_dynamic_map_beats_linear_on_values_over_several_decades():
    """The description's reason for the map: better relative error for non-uniform values.  For
    second-moment-like values spread over four decades in each block, the block-64 dynamic code
    loses far less (median relative error) than the block-64 linear absmax code."""
    rng = np.random.default_rng(10)
    v = 10.0 ** rng.uniform(-4, 0, (64, 1024)) * 1e-5
    lin = numerics.dequantize_block64(*numerics.quantize_block64(v, False), False)
    dyn = dynmap.dequantize_block64(*dynmap.quantize_block64(v, False), False)
    rl, rd = np.median(np.abs(lin - v) / v), np.median(np.abs(dyn - v) / v)
    assert rd < 0.25 * rl, (rd, rl)
