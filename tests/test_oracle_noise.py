"""Pins of the oracle's counter-based noise (O6, T > 0).

The oracle writes Philox4x64-10 out from its published definition (Salmon et
al., SC'11) with its own 64x64->128 multiply; numpy.random.Philox is an
independent library implementation of the same generator and must agree bit
for bit.  numpy's generator advances its counter by one before each block of
four outputs, so counter c - 1 in numpy gives the block of counter c."""
import numpy as np
import pytest
from scipy import stats

from oracle import oracle as O

M64 = (1 << 64) - 1


def _numpy_block(ctr, key):
    c = list(ctr)
    # step back by one (with borrow) so numpy's pre-increment lands on ctr
    for j in range(4):
        if c[j] > 0:
            c[j] -= 1
            break
        c[j] = M64
    g = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return [int(x) for x in g.random_raw(4)]


def test_philox_matches_numpy_random():
    rng = np.random.default_rng(123)
    ctrs, keys = [], []
    for _ in range(64):
        ctrs.append([int(x) for x in rng.integers(0, 2**63, 4, dtype=np.uint64)] )
        keys.append([int(x) for x in rng.integers(0, 2**63, 2, dtype=np.uint64)])
    # edge values: zero, all-ones, carries
    ctrs += [[0, 0, 0, 0], [M64, M64, M64, M64], [0, 5, 0, 0], [M64, 0, 7, 0]]
    keys += [[0, 0], [M64, M64], [1, 0], [0, 1]]
    got = O.philox4x64_10(np.array(ctrs, dtype=np.uint64), np.array(keys, dtype=np.uint64))
    for c, k, g in zip(ctrs, keys, got):
        assert [int(x) for x in g] == _numpy_block(c, k)


def test_noise_word_layout():
    seed, step, pos = 0x1234_5678_9ABC, 105, 300
    v = np.arange(40)
    w = O.noise_words(seed, step, pos, v)
    for blk in range(5):
        ref = _numpy_block([blk, pos, step, 0], [seed, 0])
        for j in range(8):
            word = ref[j >> 1]
            want = (word >> (32 * (j & 1))) & 0xFFFFFFFF
            assert int(w[blk * 8 + j]) == want
    # unordered / repeated ids give the same words
    perm = np.array([39, 0, 17, 17, 8])
    assert np.array_equal(O.noise_words(seed, step, pos, perm), w[perm])


def test_negative_and_large_keys_wrap_to_u64():
    a = O.noise_words(-1, 2**64 + 3, -5, np.arange(8))
    b = O.noise_words(M64, 3, M64 - 4, np.arange(8))
    assert np.array_equal(a, b)


def test_gumbel_transform_matches_scipy_ppf():
    w = np.array([0, 1, 2**31 - 1, 2**31, 2**32 - 2, 2**32 - 1, 123456789], dtype=np.uint64)
    u = (w.astype(np.float64) + 0.5) / 2**32
    ref = stats.gumbel_r.ppf(u).astype(np.float32)
    np.testing.assert_array_equal(O.gumbel_from_words(w), ref)
    assert np.all(np.isfinite(O.gumbel_from_words(w)))


def test_gumbel_moments():
    g = O.gumbel(7, 1, 2, np.arange(400_000)).astype(np.float64)
    assert abs(g.mean() - np.euler_gamma) < 0.01
    assert abs(g.var() - np.pi ** 2 / 6) < 0.02
    ks = stats.kstest(g, stats.gumbel_r.cdf)
    assert ks.pvalue > 1e-4


def test_noise_uncorrelated_across_keys():
    v = np.arange(100_000)
    base = O.gumbel(3, 10, 20, v).astype(np.float64)
    for other in [O.gumbel(3, 11, 20, v), O.gumbel(3, 10, 21, v), O.gumbel(4, 10, 20, v),
                  O.gumbel(3, 10, 20, v + 1)]:
        r = np.corrcoef(base, other.astype(np.float64))[0, 1]
        assert abs(r) < 5 / np.sqrt(v.size)
