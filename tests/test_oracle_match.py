"""Pins of the oracle match walk (O8) by draft-free replay (SPOT,
Propositions 1 and 2: at T = 0 state-equality verification reproduces the
draft-free trajectory; at T > 0 with noise shared between drafter and target
the transition is deterministic given the noise, so verification reduces to
state equality).

A toy target maps each block state to fp32 logits (synth.state_keyed_logits),
so equal states get equal logits as with a real model.  The draft-free decode
runs step by step; its states are planted as a chain in a random tree with
decoys; one verification step must accept exactly the planted chain and land on
the draft-free state."""
import numpy as np
import pytest

from branch_verify_amd import synth
from oracle import oracle as O

N, V, SEED = 8, 64, 21


def _decode_free(s0, T, step0, pos0, steps):
    """Draft-free decoding: one target forward and one commit per step."""
    traj = [s0.copy()]
    for t in range(steps):
        cur = traj[-1][None, :]
        rows = O.masked_rows(cur)
        if rows.size == 0:
            break
        logits = synth.state_keyed_logits(SEED, cur[0], V)[rows]
        nxt, *_ = O.commit(logits, rows, cur, np.array([-1]), T, SEED, step0 + t, pos0)
        traj.append(nxt[0].copy())
    return traj


def _plant(traj, n_decoys, rng):
    """Tree: 0 = traj[0]; planted chain j_t = traj[t] with parent j_{t-1};
    decoys off random nodes unmask one random masked position."""
    states = [traj[0]]
    parent = [-1]
    planted = [0]
    for t in range(1, len(traj)):
        parent.append(planted[-1])
        states.append(traj[t])
        planted.append(len(states) - 1)
    for _ in range(n_decoys):
        p = int(rng.integers(0, len(states)))
        row = states[p].copy()
        free = np.flatnonzero(row == O.MASK)
        if free.size == 0:
            continue
        n = int(rng.choice(free))
        row[n] = int(rng.integers(0, V))
        if any(np.array_equal(row, s) for s in traj):
            continue
        states.append(row)
        parent.append(p)
    # shuffle draft order while keeping parents before children
    B1 = len(states)
    order = [0] + list(rng.permutation(np.arange(1, B1)))
    depth = O.tree_depths(parent)
    order = [0] + sorted(order[1:], key=lambda i: (depth[i], rng.random()))
    new_index = {old: new for new, old in enumerate(order)}
    st = np.stack([states[o] for o in order]).astype(np.int32)
    par = np.array([-1] + [new_index[parent[o]] for o in order[1:]])
    return st, par, [new_index[p] for p in planted]


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("case", range(6))
def test_replay_accepts_planted_chain(T, case):
    rng = np.random.default_rng(100 + case)
    s0 = rng.integers(0, V, N).astype(np.int32)
    s0[rng.choice(N, 6, replace=False)] = O.MASK
    depth_planted = int(rng.integers(1, 5))
    step0, pos0 = 500 + case, 1000
    traj = _decode_free(s0, T, step0, pos0, depth_planted)
    st, par, planted = _plant(traj, n_decoys=int(rng.integers(2, 8)), rng=rng)
    assert O.state_violations(st, par, 1) == []
    rows = O.masked_rows(st)
    logits = np.concatenate([synth.state_keyed_logits(SEED, st[i], V)[[r - i * N for r in rows if r // N == i]]
                             for i in range(st.shape[0])])
    nxt, cpos, tok, conf, S = O.commit(logits, rows, st, par, T, SEED, step0, pos0)
    chain, h, status = O.match_tree(st, nxt, cpos, par, S_max=1)
    assert status == O.SFV_OK
    assert h == len(traj) - 1
    assert list(chain[:h]) == planted[1:]
    assert np.all(chain[h:] == -1)
    # the accepted chain plus the target's own commit equals draft-free decoding
    longer = _decode_free(s0, T, step0, pos0, h + 1)
    assert np.array_equal(O.final_state(nxt, chain, h), longer[-1])


def test_duplicate_drafts_lowest_index():
    st = np.array([[-1, -1, 3], [2, -1, 3], [2, -1, 3], [-1, 1, 3]], np.int32)
    par = np.array([-1, 0, 0, 0])
    nxt = st.copy(); nxt[0, 0] = 2
    cpos = np.array([[0], [-1], [-1], [-1]])
    chain, h, status = O.match_tree(st, nxt, cpos, par)
    assert h == 1 and chain[0] == 1 and status == O.SFV_OK


def test_miss_and_complete_block_stop():
    st = np.array([[-1, 4], [5, 4]], np.int32)
    par = np.array([-1, 0])
    nxt = np.array([[6, 4], [5, 4]], np.int32)
    chain, h, _ = O.match_tree(st, nxt, np.array([[0], [-1]]), par)
    assert h == 0 and list(chain) == [-1, -1]
    nxt = np.array([[5, 4], [5, 4]], np.int32)      # hit, then branch 1 is complete
    chain, h, _ = O.match_tree(st, nxt, np.array([[0], [-1]]), par)
    assert h == 1 and list(chain) == [1, -1]
    st_full = np.array([[1, 2], [1, 2]], np.int32)  # main branch already complete
    chain, h, _ = O.match_tree(st_full, st_full, np.array([[-1], [-1]]), par)
    assert h == 0


def test_inconsistent_draft_sets_status():
    st = np.array([[-1, -1, 3], [2, 9, 3]], np.int32)
    par = np.array([-1, 0])
    nxt = np.array([[2, 9, 3], [2, 9, 3]], np.int32)
    cpos = np.array([[0], [-1]])
    assert O.match_tree(st, nxt, cpos, par, S_max=2)[1:] == (1, O.SFV_OK)
    chain, h, status = O.match_tree(st, nxt, cpos, par, S_max=1)
    assert status == O.SFV_E_STATE and h == 0 and list(chain) == [-1, -1]


def _walk_by_levels(st, par, traj):
    """Brute force of the accepted run length: the largest k such that every
    tree level 1..k holds a draft equal to the draft-free state after that
    many steps (the walk may jump between subtrees of one level), cut where a
    trajectory state has nothing left to commit."""
    depth = O.tree_depths(par)
    k = 0
    while k + 1 < len(traj) and np.any(O.masked_rows(traj[k][None]).size > 0):
        level = [j for j in range(1, st.shape[0]) if depth[j] == k + 1]
        if not any(np.array_equal(st[j], traj[k + 1]) for j in level):
            break
        k += 1
    return k


def _mixed_depth_tree(rng, traj, B1):
    """Drafts hold draft-free states at any depth: a child copies its parent's
    trajectory state (0 new positions) or moves 1 or 2 steps along it, so the
    same state appears at depths other than its step count; a few drafts are
    one-position decoys off the trajectory."""
    st, par, t_of = [traj[0]], [-1], [0]
    while len(st) < B1:
        p = int(rng.integers(0, len(st)))
        if t_of[p] < 0 or rng.random() < 0.2:
            row = st[p].copy()
            free = np.flatnonzero(row == O.MASK)
            if free.size == 0:
                continue
            row[int(rng.choice(free))] = int(rng.integers(0, V))
            if any(np.array_equal(row, s) for s in traj):
                continue
            st.append(row); par.append(p); t_of.append(-1)
            continue
        t = min(len(traj) - 1, t_of[p] + int(rng.integers(0, 3)))
        st.append(traj[t].copy()); par.append(p); t_of.append(t)
    return np.stack(st).astype(np.int32), np.array(par)


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("case", range(12))
def test_mixed_depth_drafts_keep_the_draft_free_trajectory(T, case):
    """States of the draft-free trajectory placed at the wrong tree depth (a
    zero-position draft shifts its subtree down a level; a two-position draft
    shifts it up) must not extend the run: the final state after the step
    equals draft-free decoding for h + 1 steps (SPOT, Proposition 2 at
    T = 1, Proposition 1 at T = 0), and h is the level-by-level brute force."""
    rng = np.random.default_rng(700 + case)
    s0 = rng.integers(0, V, N).astype(np.int32)
    s0[rng.choice(N, 7, replace=False)] = O.MASK
    step0, pos0 = 60 + case, 333
    traj = _decode_free(s0, T, step0, pos0, 7)
    st, par = _mixed_depth_tree(rng, traj, B1=int(rng.integers(6, 20)))
    assert O.state_violations(st, par, 2) == []
    rows = O.masked_rows(st)
    logits = np.concatenate([synth.state_keyed_logits(SEED, st[i], V)[[r - i * N for r in rows if r // N == i]]
                             for i in range(st.shape[0])])
    nxt, cpos, tok, conf, S = O.commit(logits, rows, st, par, T, SEED, step0, pos0)
    chain, h, status = O.match_tree(st, nxt, cpos, par, S_max=2)
    assert status == O.SFV_OK
    assert h == _walk_by_levels(st, par, traj)
    depth = O.tree_depths(par)
    assert [int(depth[j]) for j in chain[:h]] == list(range(1, h + 1))
    longer = _decode_free(s0, T, step0, pos0, h + 1)
    assert np.array_equal(O.final_state(nxt, chain, h), longer[-1])


def test_two_position_draft_at_depth_one_is_not_a_second_hop():
    """Main branch, its one-step draft-free successor at depth 1, and the
    two-step successor also at depth 1 (it unmasks two positions).  The walk
    takes one hop only: continuing from the depth-1 two-step state would
    commit it with the noise of step step0 + 1 instead of step0 + 2."""
    for seed_case in range(20):
        rng = np.random.default_rng(900 + seed_case)
        s0 = rng.integers(0, V, N).astype(np.int32)
        s0[rng.choice(N, 5, replace=False)] = O.MASK
        traj = _decode_free(s0, 1.0, 7, 50, 3)
        st = np.stack([traj[0], traj[1], traj[2]]).astype(np.int32)
        par = np.array([-1, 0, 0])
        rows = O.masked_rows(st)
        logits = np.concatenate([synth.state_keyed_logits(SEED, st[i], V)[[r - i * N for r in rows if r // N == i]]
                                 for i in range(3)])
        nxt, cpos, *_ = O.commit(logits, rows, st, par, 1.0, SEED, 7, 50)
        chain, h, status = O.match_tree(st, nxt, cpos, par, S_max=2)
        assert status == O.SFV_OK and h == 1 and list(chain) == [1, -1, -1]
        assert np.array_equal(O.final_state(nxt, chain, h), traj[2])
