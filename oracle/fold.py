"""CPU oracle for SpecFold's folded verification of the same branch batch.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

[SF] SpecFold: Folding Multi-Branch Redundancy for Faster Speculative Decoding
in Diffusion Language Models -- Sec. 3.2 (the per-token parent-child gate,
Eq. 4 and 5), App. A (per-branch Q/K/V, (m, Z, O) and FFN tables inherited
from the parent and overwritten at recomputed positions), App. A.1 and Alg. 2
(the folded attention correction), App. B (gate, source resolution,
compacted recomputed lists, the folded-attention kernels).

Readings (the copy of the pages lost Eq. 4 and Alg. 2):
  * rho_{i,n} = ||H_i[n] - H_par(i)[n]||_2 / ||H_par(i)[n]||_2; position n of
    draft i folds iff rho <= delta, decided as num <= delta^2 * den in fp64
    with num = ||H_i[n] - H_par(i)[n]||^2, den = ||H_par(i)[n]||^2 and delta the
    fp32 value of the argument (so den = 0 folds only when num = 0, and a
    negative delta folds nothing).  The main branch recomputes everything.
  * The compacted recomputed list is in (branch, position) order (the pages
    fill it through atomic counters, whose order is not fixed).
  * A folded slot's query, key and value are those of its source: the
    nearest ancestor (parent chain) in which the position is recomputed.
  * The folded attention is exact with respect to the branch's own tables,
    so its plain definition is full attention of the resolved query over
    [shared context | the branch's resolved block keys].

Pins (tests/test_oracle_fold.py): a hand-worked gate example
(tests/golden/fold_gate_tiny.json), brute-force source resolution along
root paths, delta < 0 == dense attention, delta = inf gives every branch the
main branch's outputs, and the method's own hop-by-hop (m, Z, O) correction
(attention_fold_chain) equal to the definition in fp64.
"""
from __future__ import annotations

import numpy as np

from .oracle import attention, root_path


def fold_residual(H, parent):
    """num[i][n] = ||H_i[n] - H_par(i)[n]||^2 and den[i][n] = ||H_par(i)[n]||^2
    in fp64 ([SF] Sec. 3.2, Eq. 4: the relative residual between a draft's
    layer-input hidden state and its parent's at the same position).  Row 0
    (the main branch, no parent) is left NaN."""
    H = np.asarray(H, np.float64)
    B1 = H.shape[0]
    num = np.full(H.shape[:2], np.nan)
    den = np.full(H.shape[:2], np.nan)
    for i in range(1, B1):
        p = int(parent[i])
        diff = H[i] - H[p]
        num[i] = np.sum(diff * diff, axis=-1)
        den[i] = np.sum(H[p] * H[p], axis=-1)
    return num, den


def fold_gate(H, parent, delta):
    """Gate, source resolution and compaction ([SF] Sec. 3.2, Eq. 5; App. B).

    H [B1][N][D] (any float dtype), parent [B1] with parent[0] = -1, delta the
    recompute threshold (taken as fp32).  Returns
      recompute [B1][N] bool  -- position recomputed in that branch
      src       [B1][N] int   -- nearest recomputed ancestor (self if recomputed)
      rec_rows  [R] int       -- flat i*N + n of every recomputed slot, in order
      branch_off [B1+1] int   -- branch i's recomputed slots are
                                 rec_rows[branch_off[i]:branch_off[i+1]]"""
    H = np.asarray(H)
    B1, N = H.shape[:2]
    d32 = float(np.float32(delta))
    num, den = fold_residual(H, parent)
    recompute = np.ones((B1, N), dtype=bool)
    if d32 >= 0.0:
        recompute[1:] = ~(num[1:] <= (d32 * d32) * den[1:])
    # first source: self if recomputed, else the parent (App. B, the gate's
    # per-program output); then follow the sources hop by hop
    first = np.where(recompute, np.arange(B1)[:, None], np.asarray(parent)[:, None])
    src = np.empty((B1, N), dtype=np.int64)
    for i in range(B1):
        for n in range(N):
            s = int(first[i, n])
            while not recompute[s, n]:
                s = int(first[s, n])
            src[i, n] = s
    rec_rows = np.flatnonzero(recompute.reshape(-1)).astype(np.int64)
    per_branch = recompute.sum(axis=1)
    branch_off = np.concatenate([[0], np.cumsum(per_branch)]).astype(np.int64)
    return recompute, src, rec_rows, branch_off


def resolve_tables(q, k_blk, v_blk, src):
    """[SF] App. A: a branch's Q/K/V tables start as its parent's and only its
    recomputed positions are overwritten, so slot (i, n) holds the projections
    computed in branch src[i][n]."""
    q = np.asarray(q)
    k_blk = np.asarray(k_blk)
    v_blk = np.asarray(v_blk)
    B1, N = src.shape
    cols = np.arange(N)[None, :].repeat(B1, axis=0)
    return q[src, cols], k_blk[src, cols], v_blk[src, cols]


def attention_folded(q, k_blk, v_blk, k_ctx, v_ctx, src, scale):
    """Folded verification attention, by its definition ([SF] Sec. 3.2 and
    App. A.1: a folded query's output stays exact with respect to the
    branch's own KV table): attention of every resolved query over [shared
    context | the branch's resolved block keys].  Same outputs as
    oracle.attention: o [B1][N][Hq][d], lse [B1][N][Hq]."""
    qr, kr, vr = resolve_tables(q, k_blk, v_blk, src)
    return attention(qr, kr, vr, k_ctx, v_ctx, scale)


def attention_fold_chain(q, k_blk, v_blk, k_ctx, v_ctx, parent, recompute, src, scale):
    """The method's own steps ([SF] Alg. 2, App. A.1 and B), in fp64, used to
    pin attention_folded: recomputed rows take full attention over their
    branch's resolved table; a folded row (i, n) starts from its source a's
    state (m, Z, O) and walks the chain a -> ... -> i, where at each hop into
    branch c every recomputed position j of c swaps the parent's key/value
    (the parent's resolved slot j) for c's own.  m stays the source's max."""
    q = np.asarray(q, np.float64)
    k_blk = np.asarray(k_blk, np.float64)
    v_blk = np.asarray(v_blk, np.float64)
    k_ctx = np.asarray(k_ctx, np.float64)
    v_ctx = np.asarray(v_ctx, np.float64)
    B1, N, Hq, d = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    _, kr, vr = resolve_tables(q, k_blk, v_blk, src)
    o = np.empty((B1, N, Hq, d))
    lse = np.empty((B1, N, Hq))
    for i in range(B1):
        for n in range(N):
            a = int(src[i, n])
            hops = root_path(parent, i)
            hops = hops[:hops.index(a)][::-1]     # branches below a, top-down
            for h in range(Hq):
                g = h // G
                qv = q[a, n, h]
                K = np.concatenate([k_ctx[g], kr[a, :, g]])
                V = np.concatenate([v_ctx[g], vr[a, :, g]])
                s = K @ qv * scale
                m = s.max()
                e = np.exp(s - m)
                Z = e.sum()
                A = e @ V                          # Z * O
                for c in hops:
                    pc = int(parent[c])
                    for j in np.flatnonzero(recompute[c]):
                        s_old = kr[pc, j, g] @ qv * scale
                        s_new = k_blk[c, j, g] @ qv * scale
                        e_old, e_new = np.exp(s_old - m), np.exp(s_new - m)
                        A = A - e_old * vr[pc, j, g] + e_new * v_blk[c, j, g]
                        Z = Z - e_old + e_new
                o[i, n, h] = A / Z
                lse[i, n, h] = m + np.log(Z)
    return o, lse


def fold_ratio(recompute) -> float:
    """Share of draft slots (branches 1..B) that fold."""
    r = np.asarray(recompute)[1:]
    return float(1.0 - r.mean()) if r.size else 0.0
