"""Storage formats of the step, in numpy (oracle; test infrastructure only).

* bf16: decoding, round-to-nearest-even from fp32 (used for the bf16 input
  gradient dX), and the stochastic rounding of the fp32 weight to bf16.
  FORGE explainer (gist.science), Technical Summary section 2 "Precision and
  Fidelity": weight write-backs are rounded stochastically so that sub-ULP
  updates accumulate without bias instead of vanishing in bf16's dead zone.
* OCP fp8 e4m3 decoding (FORGE explainer, Technical Summary section 4
  "Composability": FORGE composes with fp8 quantisation).  Format: 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
  subnormal; S.1111.111 is NaN; there is no infinity; the largest finite
  magnitude is 448.
* Block-64 int8 optimizer moments (same section "Precision and Fidelity":
  int8 optimizer states use blocks of 64 elements instead of 2048).  Reading
  used here: blocks are 64 consecutive elements of the row-major tensor; the
  stored block scale s is the block's absmax rounded to fp32; signed moments
  use codes -127..127 and non-negative moments use 0..255; code =
  round-half-even of value * levels / s, taken in float64 from the new value;
  dequantised value = code * s / levels.  Two readings the pages leave open:
  - a non-negative (second) moment that is not zero never stores code 0: its
    code is at least 1.  Plain rounding would store about one value in eleven
    of a Gaussian block as 0, the next step's denominator would then lose that
    element's history while its first moment keeps it, and single updates
    would grow by orders of magnitude; the pages claim full-precision
    fidelity for the int8 states (section 3), which rules that out;
  - a block with scale 0 stores all-zero codes; a block holding a NaN or an
    infinity stores all-zero codes and a NaN scale, so it dequantises to NaN
    and a non-finite moment stays visible.
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x64_10

BLOCK = 64


# ----------------------------------------------------------------------------- bf16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even; NaN becomes a quiet NaN of the same sign."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return r


def sr_bits(seed: int, step: int, idx: np.ndarray) -> np.ndarray:
    """16 random bits for each weight element index idx = n*K + k.

    Element i uses Philox4x64-10 with counter (i >> 4, step, 0, 0) and key
    (seed, 0).  The 256 output bits serve 16 consecutive elements: element i
    takes bits [16*(i & 3), 16*(i & 3) + 16) of output word (i & 15) >> 2.
    """
    idx = np.asarray(idx, dtype=np.uint64)
    blk = idx >> np.uint64(4)
    j = idx & np.uint64(15)
    w = philox4x64_10(blk, np.uint64(step), np.uint64(0), np.uint64(0),
                      np.uint64(seed & 0xFFFFFFFFFFFFFFFF), np.uint64(0))
    wsel = j >> np.uint64(2)
    word = np.where(wsel == 0, w[0], np.where(wsel == 1, w[1], np.where(wsel == 2, w[2], w[3])))
    sh = (j & np.uint64(3)) * np.uint64(16)
    return ((word >> sh) & np.uint64(0xFFFF)).astype(np.uint16)


def sr_bits_block(seed: int, step: int, row0: int, col0: int, rows: int, cols: int, K: int) -> np.ndarray:
    """sr_bits for the [rows, cols] block of a row-major [., K] weight at (row0, col0).

    Same values as sr_bits on the block's flat indices; requires col0 and cols to be
    multiples of 16 so that every 16-element Philox block lies inside the block, and draws
    each Philox block once.
    """
    assert col0 % 16 == 0 and cols % 16 == 0 and K % 16 == 0
    rr = np.arange(rows, dtype=np.uint64)[:, None] + np.uint64(row0)
    bb = np.arange(cols // 16, dtype=np.uint64)[None, :] + np.uint64(col0 // 16)
    blk = (rr * np.uint64(K // 16) + bb).reshape(-1)
    w = philox4x64_10(blk, np.uint64(step), np.uint64(0), np.uint64(0),
                      np.uint64(seed & 0xFFFFFFFFFFFFFFFF), np.uint64(0))
    words = np.stack(w, axis=1)                                     # [blocks, 4] uint64
    parts = [(words >> np.uint64(16 * f)) & np.uint64(0xFFFF) for f in range(4)]
    out = np.stack(parts, axis=2).reshape(-1, 16)                   # element j: word j >> 2, field j & 3
    return out.astype(np.uint16).reshape(rows, cols)


def sr_bf16(x32: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Stochastic rounding fp32 -> bf16 with the given 16 random bits per element.

    The low 16 bits of the fp32 pattern u are the part below the bf16 ULP.
    (u + r) >> 16 rounds the magnitude up with probability (u mod 2^16)/2^16,
    so the expected result is the fp32 value.  Values that bf16 holds exactly
    and infinities are unchanged; NaN stays a NaN of the same sign.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    out = ((u + np.asarray(r16, dtype=np.uint64)) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return out


# ----------------------------------------------------------------------------- fp8 e4m3
def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3 bytes to float64 from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, f / 8.0 * 2.0 ** -6, (1.0 + f / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = sign * mag
    val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return val


# ----------------------------------------------------------------------------- int8 block-64 moments
def levels(signed: bool) -> int:
    return 127 if signed else 255


def quantize_blocks(x64: np.ndarray, signed: bool, block: int = BLOCK):
    """Quantise a [rows, cols] moment in blocks of `block` consecutive row elements (the last
    block of a row may be shorter) -> (codes, fp32 scales [rows, ceil(cols / block)])."""
    x = np.asarray(x64, dtype=np.float64)
    rows, cols = x.shape
    nb = -(-cols // block)
    xp = np.zeros((rows, nb * block))
    xp[:, :cols] = x
    xb = xp.reshape(rows, nb, block)
    finite = np.isfinite(xb).all(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        s = np.where(finite, np.max(np.abs(np.where(np.isfinite(xb), xb, 0.0)), axis=2), np.nan).astype(np.float32)
    lv = levels(signed)
    use = finite & (s > 0)
    s64 = np.where(use, s.astype(np.float64), 1.0)[..., None]
    q = np.where(use[..., None], np.rint(np.where(np.isfinite(xb), xb, 0.0) * lv / s64), 0.0)
    if signed:
        codes = np.clip(q, -127, 127).astype(np.int8)
    else:
        q = np.where(use[..., None] & (xb > 0), np.maximum(q, 1.0), q)
        codes = np.clip(q, 0, 255).astype(np.uint8)
    return np.ascontiguousarray(codes.reshape(rows, nb * block)[:, :cols]), s


def quantize_block64(x64: np.ndarray, signed: bool):
    """Quantise a [rows, cols] moment (cols % 64 == 0) -> (codes, fp32 scales[rows, cols/64])."""
    assert np.shape(x64)[1] % BLOCK == 0
    return quantize_blocks(x64, signed, BLOCK)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, signed: bool, block: int = BLOCK) -> np.ndarray:
    rows, cols = codes.shape
    s = np.repeat(scales.astype(np.float64), block, axis=1)[:, :cols]
    return codes.astype(np.float64) * s / levels(signed)


def dequantize_block64(codes: np.ndarray, scales: np.ndarray, signed: bool) -> np.ndarray:
    return dequantize_blocks(codes, scales, signed, BLOCK)
