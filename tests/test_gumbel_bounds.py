"""The commit sweep's Gumbel bounds table (branch_verify_amd/csrc/gumbel_bounds.h).

The noisy sweep screens ids with per-bucket bounds lo <= g <= hi on the exact
noise g = fl32(-ln(-ln u)) (SPOT, "Is the output exact when the target
samples?": the sampled token must be the exact Gumbel-max, Proposition 2).
These checks hold the table to the oracle's noise values and to the bucket
mapping the kernel uses; the device self-check (test_selfcheck_bounds)
covers every one of the 2^32 words on the GPU.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "branch_verify_amd", "csrc", "gen_gumbel_bounds.py")


@pytest.fixture(scope="module")
def gen():
    spec = importlib.util.spec_from_file_location("gen_gumbel_bounds", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def table(gen):
    lo, hi = gen.bounds()
    return lo, hi, gen.t_runs()


def test_header_is_the_generators_output(gen):
    with open(gen.HEADER) as f:
        assert f.read() == gen.header_text()


def test_buckets_tile_the_words(gen, table):
    lo, hi, runs = table
    H = gen.HALF_BUCKETS
    total = 0
    for b, run in enumerate(runs):
        if run is None:
            assert lo[b] == -np.inf and hi[b] == np.inf
            assert lo[H + b] == -np.inf and hi[H + b] == np.inf
            continue
        tf, tl = run
        total += 2 * (tl - tf + 1)
        # lower half: words tf .. tl; upper half: ~tl .. ~tf
        for w0, w1, idx in ((tf, tl, b), (0xFFFFFFFF - tl, 0xFFFFFFFF - tf, H + b)):
            ws = np.array([w0, w1], dtype=np.uint32)
            assert (gen.bucket_of_word(ws) == idx).all(), (b, w0, w1)
            if w0 > 0:
                assert gen.bucket_of_word(np.uint32(w0 - 1)) != idx
            if w1 < 0xFFFFFFFF:
                assert gen.bucket_of_word(np.uint32(w1 + 1)) != idx
    assert total == 2 ** 32


def test_bounds_hold_at_run_ends_and_samples(gen, table):
    lo, hi, runs = table
    H = gen.HALF_BUCKETS
    ends = []
    for run in runs:
        if run is None:
            continue
        tf, tl = run
        ends += [tf, tl, 0xFFFFFFFF - tl, 0xFFFFFFFF - tf]
    rng = np.random.default_rng(20261203)
    w = np.concatenate([np.array(ends, dtype=np.uint32),
                        rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    g = O.gumbel_from_words(w)
    b = gen.bucket_of_word(w)
    assert np.isfinite(lo[b]).all() and np.isfinite(hi[b]).all()
    assert (lo[b] <= g).all() and (g <= hi[b]).all()
    # narrow enough to screen: every non-empty bucket spans at most 0.1
    ok = np.isfinite(lo)
    assert float(np.max(hi[ok] - lo[ok])) < 0.1
    # the extreme words: u closest to 0 and to 1
    assert gen.bucket_of_word(np.uint32(0)) == 0 and gen.bucket_of_word(np.uint32(0xFFFFFFFF)) == H


def test_a_wrong_table_is_caught(gen, table):
    # swapping one bucket's bounds, or shifting the table by one bucket,
    # breaks the bounds at that bucket's run ends
    lo, hi, runs = table
    b = next(i for i, r in enumerate(runs) if r is not None and r[1] > r[0])
    tf, tl = runs[b]
    w = np.array([tf, tl], dtype=np.uint32)
    g = O.gumbel_from_words(w)
    assert not ((hi[b] <= g) & (g <= lo[b])).all()
    lo2, hi2 = np.roll(lo, 1), np.roll(hi, 1)
    bad = 0
    for r_b, run in enumerate(runs):
        if run is None or not np.isfinite(lo2[r_b]):
            continue
        ww = np.array(run, dtype=np.uint32)
        gg = O.gumbel_from_words(ww)
        bad += int(((gg < lo2[r_b]) | (gg > hi2[r_b])).any())
    assert bad > 0


def test_max_width_covers_every_bucket(gen, table):
    lo, hi, _ = table
    w = gen.max_width(lo, hi)
    ok = np.isfinite(lo)
    widths = hi[ok].astype(np.float64) - lo[ok].astype(np.float64)
    assert float(w) >= widths.max()
    assert float(np.nextafter(w, np.float32(0))) < widths.max()  # rounded up, not padded
    with open(gen.HEADER) as f:
        assert f"kGumbelMaxWidth = {gen._lit(w)};" in f.read()


def _lower_from_upper(hm, width):
    """The sweep's lower bound hm - fma(|hm|, 2^-21, 1.01 * width), one rounding
    per fp32 operation (the fma's single rounding taken in fp64, where the
    product and sum are exact)."""
    slack = np.float32(np.float32(width) * np.float32(1.01))
    d = (np.abs(hm).astype(np.float64) * 2.0 ** -21 + np.float64(slack)).astype(np.float32)
    return (hm - d).astype(np.float32)


def test_lower_bound_from_upper_bound(gen, table):
    # An id's key fl32(x + g) is at least the sweep's lower bound derived from its
    # upper bound fl32(x + hi): the widest bucket plus both fp32 roundings.
    lo, hi, _ = table
    width = gen.max_width(lo, hi)
    rng = np.random.default_rng(20261204)
    n = 1_000_000
    w = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    scale = np.float32(10.0) ** rng.integers(-2, 7, n).astype(np.float32)
    x = (rng.standard_normal(n).astype(np.float32) * scale).astype(np.float32)
    b = gen.bucket_of_word(w)
    key = (x + O.gumbel_from_words(w)).astype(np.float32)
    up = (x + hi[b]).astype(np.float32)
    assert (key <= up).all()
    assert (_lower_from_upper(up, width) <= key).all()
    # without the rounding term the bound fails at large |x|
    slack = np.float32(np.float32(width) * np.float32(1.01))
    assert ((up - slack).astype(np.float32) > key).any()
    # extreme magnitudes and subnormal logits
    xe = np.array([3e38, -3e38, 1e30, -1e30, 1e-40, -1e-40, 0.0, 65504.0, -65504.0], np.float32)
    we = rng.integers(0, 2 ** 32, (xe.size, 64), dtype=np.uint64).astype(np.uint32)
    xe = np.repeat(xe[:, None], 64, axis=1)
    with np.errstate(over="ignore"):
        ke = (xe + O.gumbel_from_words(we)).astype(np.float32)
        ue = (xe + hi[gen.bucket_of_word(we)]).astype(np.float32)
        le = _lower_from_upper(ue, width)
    assert np.isfinite(le).all() and (le <= ke).all() and (ke <= ue).all()
