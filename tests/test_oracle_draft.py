"""Pins of the drafting oracle (SPOT: stale conditionals, draft tree,
coupled-noise match; SSD-style chain, BlockSpec-style confidence tree)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import draft as Dr
from oracle import oracle as O


def _brute_topk(row, K):
    row = np.asarray(row, dtype=np.float64).copy()
    ids = []
    for _ in range(K):
        i = O.first_argmax(row)
        ids.append(i)
        row[i] = -np.inf
    return ids


@pytest.mark.parametrize("seed", range(5))
def test_topk_against_repeated_argmax(seed):
    rng = np.random.default_rng(seed)
    V = 300
    row = rng.standard_normal(V).astype(np.float32)
    if seed % 2:
        row[rng.integers(0, V, 40)] = row.max()    # ties at the top
        row[rng.integers(0, V, 40)] = np.float32(0.5)
    for K in (1, 7, 32):
        ids, vals = Dr.stale_topk(row, K)
        assert ids.tolist() == _brute_topk(row, K)
        assert np.array_equal(vals, row[ids])


def _stale_inputs(rng, N, V, K, sharp=(0.5, 8.0)):
    lg = (rng.standard_normal((N, V)) * np.exp(rng.uniform(*np.log(sharp), (N, 1)))).astype(np.float32)
    conf = np.array([np.float32(1.0 / O.confidence_sum(lg[n])) for n in range(N)], dtype=np.float32)
    ids = np.zeros((N, K), np.int64)
    vals = np.zeros((N, K), np.float32)
    for n in range(N):
        ids[n], vals[n] = Dr.stale_topk(lg[n], K)
    return lg, ids, vals, conf


def test_chain_is_confidence_order_of_stale_argmax():
    rng = np.random.default_rng(1)
    N, V, K = 12, 64, 8
    root = rng.integers(0, V, N)
    root[[0, 2, 3, 5, 7, 8, 11]] = O.MASK
    _, ids, vals, conf = _stale_inputs(rng, N, V, K)
    parent, states, nd = Dr.draft_tree(root, ids, vals, conf, D=5, W=0, T=0.0, seed=1, step0=0, pos0=0)
    order = sorted([n for n in range(N) if root[n] == O.MASK], key=lambda n: -conf[n])
    assert nd == 5 and parent.tolist() == [-1, 0, 1, 2, 3, 4]
    want = root.copy()
    for k in range(5):
        want[order[k]] = ids[order[k], 0]
        assert np.array_equal(states[k + 1], want)


@pytest.mark.parametrize("T", [0.0, 1.0, 0.6])
def test_chain_follows_a_static_target(T):
    """A target whose logits do not depend on the state commits positions in
    confidence order; the chain drafted from its stale conditionals (K = V,
    the target's own noise) is exactly its trajectory (SPOT Prop. 1-2)."""
    rng = np.random.default_rng(int(T * 10) + 3)
    N, V = 10, 48
    root = rng.integers(0, V, N)
    root[rng.choice(N, 7, replace=False)] = O.MASK
    lg, ids, vals, conf = _stale_inputs(rng, N, V, V)
    seed, step0, pos0 = 9, 50, 128
    parent, states, nd = Dr.draft_tree(root, ids, vals, conf, D=6, W=1, T=T, seed=seed, step0=step0, pos0=pos0)
    cur = root.copy()
    for t in range(6):
        rows = O.masked_rows(cur[None])
        nxt, cpos, *_ = O.commit(lg[rows % N], rows, cur[None], np.array([-1]), T, seed, step0 + t, pos0)
        cur = nxt[0]
        assert np.array_equal(states[t + 1], cur), t


def test_drafted_token_is_the_commit_token_when_k_is_v():
    rng = np.random.default_rng(2)
    V = 200
    for trial in range(20):
        row = (rng.standard_normal(V) * 2).astype(np.float32)
        ids, vals = Dr.stale_topk(row, V)
        T = [0.0, 1.0, 0.3, 2.0][trial % 4]
        tok = Dr.drafted_token(ids, vals, T, 5, 77 + trial, 300)
        assert tok == O.sample_token(row, T, 5, 77 + trial, 300)


def _brute_tree_nodes(root, conf, W):
    """Every node reachable by committing top-W positions, with its
    probability in exact rational arithmetic (fp32 confidences are exact
    rationals), so no rounding of the normaliser enters the ranking."""
    N = len(root)
    order = Dr.confidence_order(root, conf)
    cq = {n: Fraction(float(conf[n])) for n in range(N)}
    out = []

    def rec(path, P):
        masked = [n for n in range(N) if root[n] == O.MASK and n not in path]
        if not masked:
            return
        total = sum((cq[m] for m in masked), Fraction(0))
        for n in [n for n in order if n not in path][:W]:
            p = P * cq[n] / total
            out.append((p, path + (n,)))
            rec(path + (n,), p)

    rec((), Fraction(1))
    return out


@pytest.mark.parametrize("W", [1, 2, 3, 5])
def test_tree_is_the_most_probable_nodes(W):
    """Child probabilities never exceed the parent's, so best-first yields the
    D most probable reachable nodes (brute-force enumeration)."""
    rng = np.random.default_rng(10 + W)
    N, V, K = 6, 32, 4
    root = rng.integers(0, V, N)
    root[[0, 1, 3, 4, 5]] = O.MASK
    _, ids, vals, conf = _stale_inputs(rng, N, V, K)
    D = 12
    parent, states, nd = Dr.draft_tree(root, ids, vals, conf, D=D, W=W, T=0.0, seed=0, step0=0, pos0=0)
    nodes = sorted(_brute_tree_nodes(root, conf, W), key=lambda x: -x[0])
    assert nd == min(D, len(nodes))
    for p, path in nodes[:nd]:
        want = root.copy()
        for n in path:
            want[n] = ids[n, 0]
        assert any(np.array_equal(want, s) for s in states[1:nd + 1]), path
    # every draft extends its parent by one position
    for b in range(1, nd + 1):
        diff = np.flatnonzero(states[b] != states[parent[b]])
        assert diff.size == 1 and states[parent[b]][diff[0]] == O.MASK


def test_tree_probabilities_match_exact_rationals():
    """Every drafted node's probability, recomputed along its root path in
    exact rational arithmetic and rounded once, is within a few fp64 ulps per
    level of the best-first order the oracle took: the oracle's normaliser is
    the exact sum rounded once, so equal sets of confidences give equal
    normalisers in any position order."""
    rng = np.random.default_rng(31)
    N, V, K = 12, 40, 4
    root = rng.integers(0, V, N)
    root[rng.choice(N, 9, replace=False)] = O.MASK
    _, ids, vals, conf = _stale_inputs(rng, N, V, K)
    conf[[1, 4, 7]] = conf[0]                       # equal confidences at several positions
    parent, states, nd = Dr.draft_tree(root, ids, vals, conf, D=30, W=3, T=0.0, seed=0, step0=0, pos0=0)
    exact = {0: Fraction(1)}
    for b in range(1, nd + 1):
        u = int(parent[b])
        masked = [m for m in range(N) if states[u][m] == O.MASK]
        n = int(np.flatnonzero(states[b] != states[u])[0])
        exact[b] = exact[u] * Fraction(float(conf[n])) / sum((Fraction(float(conf[m])) for m in masked),
                                                             Fraction(0))
    # best-first: the exact probabilities never increase along the drafting order
    # by more than the rounding of the oracle's fp64 path products allows
    for b in range(2, nd + 1):
        assert float(exact[b]) <= float(exact[b - 1]) * (1 + 1e-13)
    # the fsum normaliser is order-free: a permuted position order sums the same
    masked0 = [m for m in range(N) if root[m] == O.MASK]
    vals0 = [float(conf[m]) for m in masked0]
    assert math.fsum(vals0) == math.fsum(vals0[::-1]) == float(sum(Fraction(v) for v in vals0))


def test_tree_padding_and_probabilities_decrease():
    rng = np.random.default_rng(4)
    N, V, K = 5, 16, 3
    root = rng.integers(0, V, N)
    root[[1, 3]] = O.MASK
    _, ids, vals, conf = _stale_inputs(rng, N, V, K)
    parent, states, nd = Dr.draft_tree(root, ids, vals, conf, D=9, W=2, T=0.0, seed=0, step0=0, pos0=0)
    assert nd == 4          # root+a, root+b, root+a+b (twice: from either side)
    assert parent[5:].tolist() == [0] * 5
    for b in range(5, 10):
        assert np.array_equal(states[b], root)
