"""GPU parity of drafting from stale conditionals against the CPU oracle,
through the C ABI: top-K ids and logits bit-exact; draft trees (parents,
states, draft count) equal to the oracle's on the same seeded inputs, or
differing from it only where two best-first candidates' probabilities are
within TIE_REL of each other; and a drafted chain fully accepted by a
state-independent target at T = 0 and T > 0.

TIE_REL.  The kernel sums a node's normaliser as a fixed pairwise fp64 tree
over 256 leaves, the oracle as the exact sum rounded once (math.fsum).  Per
tree level the two probabilities P(u) c_n / sum c_m then differ by at most
(8 + 0.5 + 4) fp64 roundings (the pairwise levels, the rounding of the exact
sum, a multiply and a divide on each side), so by at most 63 * 12.5 * 2^-53
< 1e-13 relative at the deepest tree (63 drafts).  A best-first choice can
therefore differ only between candidates within 2e-13 of each other; 1e-12
is used."""
import math
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import sfv, synth
from branch_verify_amd.step import VerifyStep
from oracle import draft as Dr
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_topk(lg, rows, conf, N, branch, K):
    M, V = lg.shape
    ids = torch.full((N, K), -7, dtype=torch.int32, device="cuda")
    vals = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    cpos = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    wsb = sfv.sfv_stale_topk_workspace_bytes(M, V, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    sfv.sfv_stale_topk(_dev(lg), _dev(rows.astype(np.int32)), _dev(conf), M, V, N, branch, K, ids, vals, cpos,
                       ws, wsb)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy(), cpos.cpu().numpy()


@pytest.mark.parametrize("V,K", [(151936, 32), (4096, 7), (64, 32), (33, 1)])
def test_stale_topk_parity(gpu_lib, V, K):
    rng = np.random.default_rng(V + K)
    B1, N = 3, 24
    st = rng.integers(0, V, (B1, N)).astype(np.int32)
    st[rng.random((B1, N)) < 0.5] = -1
    st[1, :5] = -1
    rows = O.masked_rows(st)
    M = rows.size
    lg = synth.draw_logits(M, V, 7)
    br1 = [r for r in range(M) if rows[r] // N == 1]
    lg[br1[0]] = 0.25                                   # constant row: the many-ties fallback
    lg[br1[1], rng.integers(0, V, 50)] = lg[br1[1]].max() + 1.0   # ties at the top
    lg[br1[2], :] = np.round(lg[br1[2]], 1)             # heavy ties everywhere
    conf = rng.random(M).astype(np.float32)
    say(f"stale top-K V={V} K={K}")
    ids, vals, cpos = run_topk(lg, rows, conf, N, 1, K)
    for r in br1:
        n = rows[r] % N
        want_ids, want_vals = Dr.stale_topk(lg[r], K)
        assert np.array_equal(ids[n], want_ids), (r, n)
        assert np.array_equal(vals[n], want_vals)
        assert cpos[n] == conf[r]
    untouched = [n for n in range(N) if st[1, n] != -1]
    assert np.all(ids[untouched] == -7)


def _tree_inputs(rng, N, V, K, frac):
    root = rng.integers(0, V, N).astype(np.int32)
    root[rng.random(N) < frac] = -1
    lg = synth.draw_logits(N, V, int(rng.integers(1 << 30)))
    ids = np.zeros((N, K), np.int32)
    vals = np.zeros((N, K), np.float32)
    for n in range(N):
        i, v = Dr.stale_topk(lg[n], K)
        ids[n], vals[n] = i, v
    conf = np.array([np.float32(1.0 / O.confidence_sum(lg[n])) for n in range(N)], dtype=np.float32)
    conf[rng.integers(0, N, 3)] = conf[0]              # equal confidences: position order decides
    return root, ids, vals, conf


def run_tree(root, ids, vals, conf, D, W, T, seed, step0, pos0):
    N, K = ids.shape
    parent = torch.full((D + 1,), -9, dtype=torch.int32, device="cuda")
    states = torch.full((D + 1, N), -9, dtype=torch.int32, device="cuda")
    nd = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    sfv.sfv_draft_tree(_dev(root), _dev(ids), _dev(vals), _dev(conf), N, K, D, W, T, seed, step0, pos0,
                       parent, states, nd)
    torch.cuda.synchronize()
    return parent.cpu().numpy(), states.cpu().numpy(), int(nd.item())


TIE_REL = 1e-12


def check_tree(root, ids, vals, conf, D, W, T, seed, step0, pos0, p, s, nd):
    """The kernel's tree against the oracle's.  Equal: done.  Otherwise it is
    replayed best-first with the oracle's probabilities: every node must be a
    live candidate (a top-W masked position of its parent, by the oracle's
    confidence order) within TIE_REL of the best live candidate, carry the
    oracle's drafted token, and the tree must stop exactly when the oracle's
    rule does.  Returns the number of steps that took a near-tied
    candidate other than the oracle's."""
    p_ref, s_ref, nd_ref = Dr.draft_tree(root, ids, vals, conf, D, W, T, seed, step0, pos0)
    if nd == nd_ref and np.array_equal(p, p_ref) and np.array_equal(s, s_ref):
        return 0
    N = root.shape[0]
    W1 = max(W, 1)
    order = Dr.confidence_order(root, conf)
    prob, depth, cand = {0: 1.0}, {0: 0}, {}

    def offer(u):
        masked = [m for m in range(N) if s[u][m] == O.MASK]
        if not masked:
            return
        total = math.fsum(float(conf[m]) for m in masked)
        for n in [n for n in order if s[u][n] == O.MASK][:W1]:
            cand[(u, n)] = (prob[u] * float(conf[n])) / total

    offer(0)
    assert np.array_equal(s[0], root) and p[0] == -1
    deviations = 0
    for b in range(1, nd + 1):
        u = int(p[b])
        assert 0 <= u < b
        diff = np.flatnonzero(s[b] != s[u])
        assert diff.size == 1, b
        n = int(diff[0])
        assert (u, n) in cand, (b, u, n)
        best_key = min(cand, key=lambda k: (-cand[k], k[0], k[1]))
        assert cand[(u, n)] >= cand[best_key] * (1 - TIE_REL), (b, cand[(u, n)], cand[best_key])
        deviations += (u, n) != best_key
        assert s[b][n] == Dr.drafted_token(ids[n], vals[n], T, seed, step0 + depth[u], pos0 + n)
        prob[b], depth[b] = cand.pop((u, n)), depth[u] + 1
        offer(b)
    assert nd == D or not cand
    for b in range(nd + 1, D + 1):
        assert p[b] == 0 and np.array_equal(s[b], root)
    assert deviations > 0      # a differing tree must have taken some near-tied candidate
    return deviations


@pytest.mark.parametrize("N,V,K,D,W,T", [
    (32, 151936, 32, 8, 0, 0.0), (32, 151936, 32, 20, 4, 0.0), (32, 4096, 32, 20, 4, 1.0),
    (64, 2048, 16, 63, 16, 0.7), (8, 512, 8, 63, 3, 1.0), (256, 1024, 32, 63, 2, 0.0),
    (16, 300, 32, 0, 1, 0.0), (5, 64, 4, 10, 16, 2.0), (1, 64, 4, 3, 1, 0.0),
])
def test_draft_tree_parity(gpu_lib, N, V, K, D, W, T):
    rng = np.random.default_rng(N * 131 + D + W)
    root, ids, vals, conf = _tree_inputs(rng, N, V, K, 0.6)
    seed, step0, pos0 = 11, 200 + D, 4096
    say(f"draft tree N={N} K={K} D={D} W={W} T={T} masked={int((root == -1).sum())}")
    p, s, nd = run_tree(root, ids, vals, conf, D, W, T, seed, step0, pos0)
    dev = check_tree(root, ids, vals, conf, D, W, T, seed, step0, pos0, p, s, nd)
    say(f"draft tree: {nd} drafts, {dev} near-tie choices differ from the oracle's")


@pytest.mark.parametrize("T", [0.0, 1.0, 0.5])
def test_drafted_chain_is_accepted_by_a_static_target(gpu_lib, T):
    """Commit on the root, stale top-K and confidences from that pass, a GPU
    chain of D drafts, then one verify pass over the chain: a target whose
    logits do not depend on the state accepts every draft (K = V, coupled
    noise)."""
    rng = np.random.default_rng(int(T * 10) + 40)
    N, V, D = 16, 32, 6
    root = rng.integers(0, V, N).astype(np.int32)
    root[rng.choice(N, 10, replace=False)] = -1
    L = synth.draw_logits(N, V, 99)                  # position n's logits in every state
    S = sorted(O.confidence_sum(L[n]) for n in range(N) if root[n] == -1)
    assert min(b / a - 1 for a, b in zip(S, S[1:])) > 1e-4   # no near-ties in the commit order
    seed, step0, pos0 = 21, 500, 64
    # pass 1: the target on the root alone
    s1 = VerifyStep(1, N, 0, 1, 1, 32, 64, V, int((root == -1).sum()), [-1], T, seed, step0, pos0, S_max=-1)
    x1 = {"state": _dev(root[None])}
    s1.masked_rows(x1)
    rows1 = O.masked_rows(root[None])
    lg1 = _dev(L[rows1 % N])
    s1.commit(x1, logits=lg1)
    ids = torch.zeros((N, V), dtype=torch.int32, device="cuda")
    vals = torch.zeros((N, V), dtype=torch.float32, device="cuda")
    cpos = torch.zeros((N,), dtype=torch.float32, device="cuda")
    Kt = V if V <= 32 else 32
    wsb = sfv.sfv_stale_topk_workspace_bytes(s1.M, V, N, Kt)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    sfv.sfv_stale_topk(lg1, s1.rows, s1.conf, s1.M, V, N, 0, Kt, ids, vals, cpos, ws, wsb)
    parent = torch.zeros((D + 1,), dtype=torch.int32, device="cuda")
    states = torch.zeros((D + 1, N), dtype=torch.int32, device="cuda")
    nd = torch.zeros((1,), dtype=torch.int32, device="cuda")
    sfv.sfv_draft_tree(x1["state"][0], ids, vals, cpos, N, V, D, 1, T, seed, step0, pos0, parent, states, nd)
    torch.cuda.synchronize()
    assert int(nd.item()) == D
    par = parent.cpu().numpy()
    st = states.cpu().numpy()
    # pass 2: verify the drafted chain
    rows2 = O.masked_rows(st)
    s2 = VerifyStep(D + 1, N, 0, 1, 1, 32, 64, V, rows2.size, par, T, seed, step0, pos0, S_max=1)
    x2 = {"state": _dev(st)}
    s2.masked_rows(x2)
    s2.commit(x2, logits=_dev(L[rows2 % N]))
    s2.match(x2)
    torch.cuda.synchronize()
    h = int(s2.n_accepted.item())
    say(f"static target T={T}: {h} of {D} drafts accepted")
    assert h == D and np.array_equal(s2.chain.cpu().numpy()[:D], np.arange(1, D + 1))
