"""Dynamic (non-linear) 8-bit map for block-64 optimizer moments (oracle; test infrastructure only).

FORGE explainer (gist.science), Technical Summary section 2 "Precision and Fidelity": int8
optimizer states in blocks of 64 rather than the 2048 of common 8-bit optimizers.  Those common
optimizers (Dettmers et al., "8-bit Optimizers via Block-wise Quantization", 2022) store each
block's values normalised by the block absmax in a non-linear "dynamic tree" code: a sign bit,
then a run of zero bits whose length E is a decimal exponent, an indicator bit set to one, and
the remaining F bits a linear fraction; for non-negative tensors the sign bit is used as one more
bit of the code.  The explainer pages describe only the linear absmax code, so this map is the
comparison format, written here from that description.  Readings where the description leaves
choices (listed with the other readings of the pages):

  * signed codes (first moment): bit 7 sign, bits 6..0 the magnitude pattern p; unsigned codes
    (second moment): all 8 bits are p.  p = 0 means 0.  Otherwise E = the number of leading
    zeros of p (0..6 signed, 0..7 unsigned), F = 6 - E (signed) or 7 - E (unsigned), f = the
    low F bits of p, and the magnitude is 10^-E * (0.1 + 0.9 * (f + 1) / 2^F): the F fraction
    bits split the decade (10^-(E+1), 10^-E] into 2^F equal steps, so the top code is exactly
    1 (the block absmax) and the smallest non-zero magnitude is 10^-6 (signed) or 10^-7
    (unsigned) of it;
  * encoding takes the nearest magnitude (ties to the smaller one) of |x| / s, s the block
    absmax rounded to fp32; as for the linear map, a non-zero unsigned value never stores
    0 (it takes the smallest magnitude), and a block holding a NaN or an infinity stores zero
    codes and a NaN scale.
"""
from __future__ import annotations

import numpy as np

from .numerics import BLOCK


def magnitude_bits(signed: bool) -> int:
    return 7 if signed else 8


def code_magnitudes(signed: bool) -> np.ndarray:
    """Magnitude (relative to the block absmax) of every magnitude pattern p = 0 .. 2^B - 1."""
    B = magnitude_bits(signed)
    out = np.zeros(1 << B)
    for p in range(1, 1 << B):
        E = B - p.bit_length()                 # leading zeros within the B-bit field
        F = B - 1 - E
        f = p & ((1 << F) - 1)
        out[p] = 10.0 ** (-E) * (0.1 + 0.9 * (f + 1) / 2.0 ** F)
    return out


def decode_codes(codes: np.ndarray, signed: bool) -> np.ndarray:
    """Relative values (in [-1, 1] or [0, 1]) of stored codes."""
    mags = code_magnitudes(signed)
    c = np.asarray(codes).astype(np.int64) & 0xFF
    if signed:
        return np.where(c & 0x80, -1.0, 1.0) * mags[c & 0x7F]
    return mags[c]


def encode_relative(y: np.ndarray, signed: bool) -> np.ndarray:
    """Codes of relative values y (|y| <= 1): nearest magnitude, ties to the smaller one."""
    mags = code_magnitudes(signed)
    order = np.argsort(mags, kind="stable")            # mags[0] = 0 first
    sm = mags[order]
    mid = 0.5 * (sm[:-1] + sm[1:])                     # decision points between neighbours
    a = np.abs(np.asarray(y, np.float64))
    k = np.searchsorted(mid, a, side="left")           # a == mid -> the smaller neighbour
    p = order[k].astype(np.int64)
    if not signed:
        p = np.where((a > 0) & (p == 0), order[1], p)  # non-zero never stores 0
        return p.astype(np.uint8)
    sign = np.where(np.asarray(y) < 0, 0x80, 0)
    return np.where(p == 0, 0, p | sign).astype(np.uint8).view(np.int8)


def quantize_blocks(x64: np.ndarray, signed: bool, block: int = BLOCK):
    """[rows, cols] in blocks of `block` consecutive row elements (the last block of a row may be
    shorter) -> (codes int8/uint8, fp32 block absmax [rows, ceil(cols / block)])."""
    x = np.asarray(x64, dtype=np.float64)
    rows, cols = x.shape
    nb = -(-cols // block)
    xp = np.zeros((rows, nb * block))
    xp[:, :cols] = x
    xb = xp.reshape(rows, nb, block)
    finite = np.isfinite(xb).all(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        s = np.where(finite, np.max(np.abs(np.where(np.isfinite(xb), xb, 0.0)), axis=2), np.nan).astype(np.float32)
    use = finite & (s > 0)
    s64 = np.where(use, s.astype(np.float64), 1.0)[..., None]
    y = np.where(use[..., None], np.where(np.isfinite(xb), xb, 0.0) / s64, 0.0)
    codes = encode_relative(y, signed)
    codes = np.where(use[..., None], codes, 0).astype(np.int8 if signed else np.uint8)
    return np.ascontiguousarray(codes.reshape(rows, nb * block)[:, :cols]), s


def quantize_block64(x64: np.ndarray, signed: bool):
    """[rows, cols] (cols % 64 == 0) -> (codes int8/uint8, fp32 block absmax [rows, cols/64])."""
    assert np.shape(x64)[1] % BLOCK == 0
    return quantize_blocks(x64, signed, BLOCK)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, signed: bool, block: int = BLOCK) -> np.ndarray:
    rows, cols = codes.shape
    s = np.repeat(scales.astype(np.float64), block, axis=1)[:, :cols]
    return decode_codes(codes, signed) * s


def dequantize_block64(codes: np.ndarray, scales: np.ndarray, signed: bool) -> np.ndarray:
    return dequantize_blocks(codes, scales, signed, BLOCK)
