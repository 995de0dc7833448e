"""Pins of the oracle commit (O6, O7).

T = 0 reduces to greedy argmax (numpy.argmax returns the first maximum);
max-softmax confidence against scipy.special.softmax; Gumbel-max token
frequencies against softmax(l / T) by a chi-square test; T -> 0+ with a clear
gap equals greedy; unmask order and tie-breaks on hand-built rows."""
import numpy as np
import pytest
from scipy import special, stats

from oracle import oracle as O


def test_greedy_is_numpy_argmax():
    rng = np.random.default_rng(0)
    for _ in range(50):
        row = rng.standard_normal(1000).astype(np.float32)
        assert O.sample_token(row, 0.0, 1, 2, 3) == int(np.argmax(row))
    row = np.zeros(10, np.float32); row[[3, 7]] = 2.0
    assert O.sample_token(row, 0.0, 1, 2, 3) == 3 == int(np.argmax(row))


def test_confidence_is_softmax_max():
    rng = np.random.default_rng(1)
    for scale in [0.1, 1.28, 11.3]:
        row = (rng.standard_normal(5000) * scale).astype(np.float32)
        S = O.confidence_sum(row)
        ref = special.softmax(row.astype(np.float64)).max()
        assert abs(1.0 / S - ref) <= 1e-12 * ref


def test_gumbel_max_frequencies_chi_square():
    logits = np.array([1.0, 0.0, -1.0, 0.5, 2.0, -3.0], dtype=np.float32)
    for T in [1.0, 0.5]:
        draws = 20000
        counts = np.zeros(6)
        for step in range(draws):
            counts[O.sample_token(logits, T, 99, step, 0)] += 1
        p = special.softmax(logits.astype(np.float64) / T)
        chi2 = stats.chisquare(counts, draws * p)
        assert chi2.pvalue > 1e-4, (T, counts, draws * p)


def test_small_temperature_is_greedy():
    rng = np.random.default_rng(2)
    for s in range(20):
        row = rng.standard_normal(512).astype(np.float32)
        row[rng.integers(512)] = row.max() + 1.0
        assert O.sample_token(row, 1e-3, 5, s, 1) == int(np.argmax(row))


def test_noise_is_shared_by_step_and_position_only():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(300).astype(np.float32)
    a = O.sample_token(row, 1.0, 11, 40, 7)
    assert a == O.sample_token(row.copy(), 1.0, 11, 40, 7)
    toks = {O.sample_token(row, 1.0, 11, st, 7) for st in range(40)}
    assert len(toks) > 3


def test_key_tie_goes_to_lower_vocab_id():
    V, seed, step, pos = 64, 3, 9, 4
    g = O.gumbel(seed, step, pos, np.arange(V))
    row = np.full(V, -30.0, dtype=np.float32)
    v1, v2 = 11, 40
    row[v1] = 5.0
    key1 = np.float32(row[v1] + g[v1])
    l2 = np.float32(key1 - g[v2])
    for _ in range(8):      # nudge l2 until its key equals key1 exactly
        k2 = np.float32(l2 + g[v2])
        if k2 == key1:
            break
        l2 = np.nextafter(l2, np.float32(np.inf) if k2 < key1 else np.float32(-np.inf))
    assert np.float32(l2 + g[v2]) == key1
    row[v2] = l2
    assert O.sample_token(row, 1.0, seed, step, pos) == v1
    row2 = row.copy(); row2[[v1, v2]] = row[[v2, v1]]   # swap which id holds which logit
    # now id 11 holds l2 (key differs) and id 40 holds 5.0: the tie is gone or not,
    # but the result must be the id with the larger exact key, lower on ties
    keys = (row2 * np.float32(1.0)).astype(np.float32) + g
    want = int(np.flatnonzero(keys == keys.max())[0])
    assert O.sample_token(row2, 1.0, seed, step, pos) == want


def _commit_case():
    # three branches, N = 4, V = 8; hand-built logits
    state = np.array([[-1, -1, 2, -1],
                      [-1, 5, 2, -1],
                      [1, 1, 1, 1]], dtype=np.int32)
    parent = np.array([-1, 0, 0])
    rows = O.masked_rows(state)           # 0,1,3,4,7
    logits = np.zeros((rows.size, 8), np.float32)
    logits[0, 6] = 3.0                     # (0,0): S = 1 + 7 e^-3
    logits[1, 2] = 5.0                     # (0,1): most confident in branch 0
    logits[2, 2] = 5.0                     # (0,3): identical row to (0,1) -> tie, lower n wins
    logits[3, 1] = 1.0                     # (1,0)
    logits[4, 7] = 4.0                     # (1,3): most confident in branch 1
    return state, parent, rows, logits


def test_unmask_argmax_and_ties():
    state, parent, rows, logits = _commit_case()
    nxt, cpos, tok, conf, S = O.commit(logits, rows, state, parent, 0.0, 1, 100, 64)
    assert list(tok) == [6, 2, 2, 1, 7]
    assert S[1] == S[2]
    assert list(cpos[:, 0]) == [1, 3, -1]
    assert list(nxt[0]) == [-1, 2, 2, -1]
    assert list(nxt[1]) == [-1, 5, 2, 7]
    assert list(nxt[2]) == [1, 1, 1, 1]
    np.testing.assert_allclose(conf, [special.softmax(r.astype(np.float64)).max() for r in logits], rtol=1e-7)


def test_threshold_multi_commit():
    state, parent, rows, logits = _commit_case()
    conf1 = 1.0 / O.confidence_sum(logits[1])
    nxt, cpos, tok, conf, S = O.commit(logits, rows, state, parent, 0.0, 1, 100, 64,
                                       k_max=3, tau=float(conf1) * 0.999)
    assert list(cpos[0]) == [1, 3, -1]      # (0,1) and its tie (0,3); (0,0) is below tau
    assert list(nxt[0]) == [-1, 2, 2, 2]
    nxt, cpos, *_ = O.commit(logits, rows, state, parent, 0.0, 1, 100, 64, k_max=3, tau=0.0)
    assert list(cpos[0]) == [1, 3, 0]


def test_noise_keyed_by_depth_and_absolute_position():
    rng = np.random.default_rng(5)
    N, V = 4, 64
    state = np.full((3, N), -1, np.int32)
    parent = np.array([-1, 0, 1])          # depths 0, 1, 2
    rows = O.masked_rows(state)
    logits = np.tile(rng.standard_normal(V).astype(np.float32), (rows.size, 1))
    _, _, tok, _, _ = O.commit(logits, rows, state, parent, 1.0, 8, 50, 1000)
    for r, row in enumerate(rows):
        i, n = divmod(int(row), N)
        assert tok[r] == O.sample_token(logits[r], 1.0, 8, 50 + i, 1000 + n)
