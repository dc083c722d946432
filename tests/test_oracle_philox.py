"""Pins of the oracle's Philox4x64-10 and of the stochastic-rounding bit stream.

Pinned against numpy.random.Philox, an independent implementation of the same
published generator.  numpy advances its 256-bit counter before producing a
block, so the block for counter c is drawn from Philox(counter=c - 1).
"""
import numpy as np
import pytest

from oracle import numerics, philox


def _numpy_block(ctr, key):
    cint = sum(int(c) << (64 * i) for i, c in enumerate(ctr))
    kint = int(key[0]) | (int(key[1]) << 64)
    bg = np.random.Philox(counter=(cint - 1) % (1 << 256), key=kint)
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("seed", range(6))
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    ctr = [int(x) for x in rng.integers(0, 2 ** 64, 4, dtype=np.uint64)]
    key = [int(x) for x in rng.integers(0, 2 ** 64, 2, dtype=np.uint64)]
    got = philox.philox4x64_10(*[np.uint64(c) for c in ctr], np.uint64(key[0]), np.uint64(key[1]))
    assert [int(x) for x in got] == _numpy_block(ctr, key)


def test_philox_edge_counters():
    for ctr, key in [([0, 0, 0, 0], [0, 0]), ([2 ** 64 - 1] * 4, [2 ** 64 - 1] * 2), ([1, 0, 0, 0], [0, 0])]:
        got = philox.philox4x64_10(*[np.uint64(c) for c in ctr], np.uint64(key[0]), np.uint64(key[1]))
        assert [int(x) for x in got] == _numpy_block(ctr, key)


def test_philox_vectorised_equals_scalar():
    c0 = np.arange(1000, dtype=np.uint64) * np.uint64(7919)
    v = philox.philox4x64_10(c0, np.uint64(5), np.uint64(0), np.uint64(0), np.uint64(123), np.uint64(0))
    for i in (0, 1, 500, 999):
        s = philox.philox4x64_10(c0[i], np.uint64(5), np.uint64(0), np.uint64(0), np.uint64(123), np.uint64(0))
        assert [int(w[i]) for w in v] == [int(x) for x in s]


@pytest.mark.parametrize("seed,step", [(0x5EED0000, 1), (12345, 7), (2 ** 64 - 1, 2 ** 40)])
def test_sr_bits_match_numpy_blocks(seed, step):
    """Element i takes 16-bit field (i & 3) of word (i & 15) >> 2 of block i >> 4."""
    idx = np.concatenate([np.arange(64, dtype=np.uint64), np.uint64(2 ** 31) + np.arange(32, dtype=np.uint64)])
    bits = numerics.sr_bits(seed, step, idx)
    for i, b in zip(idx.tolist(), bits.tolist()):
        words = _numpy_block([i >> 4, step, 0, 0], [seed, 0])
        j = i & 15
        assert b == (words[j >> 2] >> (16 * (j & 3))) & 0xFFFF


def test_sr_bits_uniform_and_step_independent():
    idx = np.arange(1 << 20, dtype=np.uint64)
    a = numerics.sr_bits(77, 1, idx).astype(np.int64)
    b = numerics.sr_bits(77, 2, idx).astype(np.int64)
    # chi-square of the top 8 bits over 256 bins (df 255): 99.99% quantile is about 360
    for r in (a >> 8, b >> 8, a & 0xFF):
        hist = np.bincount(r, minlength=256)
        exp = len(r) / 256.0
        chi2 = float(((hist - exp) ** 2 / exp).sum())
        assert chi2 < 360.0, chi2
    # independence across steps and across neighbouring elements
    for x, y in ((a, b), (a[:-1], a[1:]), (a[:-16], a[16:])):
        c = np.corrcoef(x.astype(np.float64), y.astype(np.float64))[0, 1]
        assert abs(c) < 5.0 / np.sqrt(len(x)), c
    # different seeds give different streams
    assert np.mean(numerics.sr_bits(78, 1, idx[:4096]) == a[:4096]) < 0.01


@pytest.mark.parametrize("row0,col0,rows,cols,K", [(0, 0, 3, 48, 64), (5, 16, 7, 32, 128), (1000, 4080, 2, 16, 4096)])
def test_sr_bits_block_equals_per_element(row0, col0, rows, cols, K):
    idx = ((np.arange(rows, dtype=np.uint64)[:, None] + np.uint64(row0)) * np.uint64(K)
           + np.arange(cols, dtype=np.uint64)[None, :] + np.uint64(col0))
    a = numerics.sr_bits(0xABCDEF, 9, idx)
    b = numerics.sr_bits_block(0xABCDEF, 9, row0, col0, rows, cols, K)
    np.testing.assert_array_equal(a, b)
