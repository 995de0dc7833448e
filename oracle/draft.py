"""CPU oracle for drafting a tree of block states from stale conditionals.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

[SPOT] On the SPOT: Enhancing Speculative Decoding for Diffusion Language
Models via Commit-Order Prediction -- "Important context" (stale
conditionals: the latest target distributions at a block's masked positions;
draft tree: block states grown by repeatedly predicting the next committed
position, high-probability branches first, up to a budget of D drafted
states; coupled-noise match: the drafter applies the target's Gumbel noise),
"How does SPOT draft and verify?" (the drafter reads the stale top-32
probabilities at each masked position) and "How does SPOT differ from Spiffy,
SSD and BlockSpec?" (an SSD-style chain orders positions by confidence; a
BlockSpec-style tree ranks positions by the stale confidences).

Readings (the pages name the two baselines but give no algorithm):
  * Stale conditionals of position n: its top-K vocabulary ids by logit
    (ties to the lower id) with their fp32 logits, and its confidence c_n
    (the fp32 max-softmax probability of the full row).
  * Chain: the masked positions in confidence order (c descending, ties to
    the lower position); draft k commits the k-th of them to draft k-1
    (parent k-1).
  * Tree: the next-position distribution at a node u is the confidences of
    u's masked positions normalised over them; a child u+n has probability
    P(u) * c_n / sum_{m masked in u} c_m, every step in fp64, the sum being
    the exact sum of the fp64 confidences rounded once (math.fsum), which
    depends on no order (the pages fix none).  A node offers its W most
    confident masked positions as children.  Nodes are added best-first: the highest
    probability candidate, ties to the lower parent index, then the lower
    position, until D drafts or no candidate remains.  W = 1 is the chain.
  * Drafted token of position n in a child of a node at depth d: T = 0, the
    stale argmax (top-1 id); T > 0, the Gumbel-max over the K candidates with
    the target's own key fl32(fl32(l * invT) + g(seed, step0 + d, pos0 + n,
    v)), ties to the lower id (the target commits from a depth-d state with
    noise step step0 + d).
  * With fewer than D candidates, the remaining branches are copies of the
    root (parent 0): a copy adds nothing and never matches a commit.

Pins (tests/test_oracle_draft.py): top-K against repeated first-argmax
removal; chain = best-first tree with W = 1; with a state-independent toy
target the T = 0 chain equals the target's own commit trajectory (oracle
commit); with K = V the drafted T > 0 token equals the commit rule's token;
tree order against brute-force enumeration on tiny blocks in exact rational
arithmetic.
"""
from __future__ import annotations

import math

import numpy as np

from .oracle import MASK, gumbel


def stale_topk(logits_row, K: int):
    """Top-K ids of one fp32 logit row by value, ties to the lower id, and
    their values."""
    lr = np.asarray(logits_row, dtype=np.float32)
    order = np.lexsort((np.arange(lr.shape[0]), -lr.astype(np.float64)))
    ids = order[:K].astype(np.int64)
    return ids, lr[ids]


def drafted_token(top_ids, top_logit, T: float, seed: int, step: int, pos: int) -> int:
    """Token a draft commits at a position (see module readings)."""
    top_ids = np.asarray(top_ids, dtype=np.int64)
    top_logit = np.asarray(top_logit, dtype=np.float32)
    if T == 0.0:
        return int(top_ids[0])
    inv_t = np.float32(1.0) / np.float32(T)
    g = gumbel(seed, step, pos, top_ids)
    key = ((top_logit * inv_t).astype(np.float32) + g).astype(np.float32)
    best = None
    for k in range(top_ids.shape[0]):
        if best is None or key[k] > key[best] or (key[k] == key[best] and top_ids[k] < top_ids[best]):
            best = k
    return int(top_ids[best])


def confidence_order(root, conf):
    """Masked positions of the root, c descending, ties to the lower position."""
    masked = [n for n in range(len(root)) if root[n] == MASK]
    return sorted(masked, key=lambda n: (-float(np.float32(conf[n])), n))


def draft_tree(root, top_ids, top_logit, conf, D: int, W: int, T: float, seed: int,
               step0: int, pos0: int):
    """Best-first draft tree from one root state.

    root [N] int; top_ids, top_logit [N][K] (rows of unmasked positions are
    ignored); conf [N] fp32.  W = 0 means the chain (same as W = 1).
    Returns parent [D+1], states [D+1][N], n_drafts."""
    root = np.asarray(root)
    N = root.shape[0]
    conf = np.asarray(conf, dtype=np.float32)
    W = 1 if W <= 0 else W
    order = confidence_order(root, conf)
    states = [root.copy()]
    parent = [-1]
    depth = [0]
    prob = [1.0]
    cand = []  # (P, parent index, position)

    def offer(u):
        masked_u = [n for n in range(N) if states[u][n] == MASK]
        if not masked_u:
            return
        total = math.fsum(float(conf[m]) for m in masked_u)
        ranked = [n for n in order if states[u][n] == MASK][:W]
        for n in ranked:
            cand.append(((prob[u] * float(conf[n])) / total, u, n))

    offer(0)
    while len(states) < D + 1 and cand:
        k = min(range(len(cand)), key=lambda c: (-cand[c][0], cand[c][1], cand[c][2]))
        p, u, n = cand.pop(k)
        child = states[u].copy()
        child[n] = drafted_token(top_ids[n], top_logit[n], T, seed, step0 + depth[u], pos0 + n)
        states.append(child)
        parent.append(u)
        depth.append(depth[u] + 1)
        prob.append(p)
        offer(len(states) - 1)
    n_drafts = len(states) - 1
    while len(states) < D + 1:
        states.append(root.copy())
        parent.append(0)
    return np.array(parent, dtype=np.int64), np.stack(states), n_drafts
