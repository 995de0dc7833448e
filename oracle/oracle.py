"""CPU oracle for one multi-branch draft-verification step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

Plain, slow and meant to be read against the pages:

  [SF]   SpecFold: Folding Multi-Branch Redundancy for Faster Speculative
         Decoding in Diffusion Language Models.
  [SPOT] On the SPOT: Enhancing Speculative Decoding for Diffusion Language
         Models via Commit-Order Prediction.

Floating point is fp64 unless a step fixes fp32 (the logits handed to the
commit rule and the Gumbel key).  Pins (tests/test_oracle_*.py):
  tree/states   invariants by construction, planted violations
  attention     split+merge form == full form (brute force), closed forms,
                torch CPU scaled_dot_product_attention in fp64
  lm_head       brute-force loops, one-hot rows, torch CPU matmul
  philox        numpy.random.Philox (library implementation of the same
                generator), bit-exact
  gumbel        scipy.stats.gumbel_r.ppf
  commit        numpy.argmax at T = 0, scipy softmax for the confidence,
                chi-square of Gumbel-max frequencies, T -> 0+ equals greedy
  match         draft-free replay with a toy target (Prop. 1 and 2)
"""
from __future__ import annotations

import numpy as np

MASK = -1
SFV_OK = 0
SFV_E_STATE = -4

# ----------------------------------------------------------------------------
# O1, O2 — draft tree and block states
# ----------------------------------------------------------------------------


def tree_depths(parent) -> np.ndarray:
    """Depth of each branch.  [SF] introduction, Fig. 1-(b): branch 0 is the
    main branch (root) and every draft i has a parent index in {0..i-1}, so
    every parent chain reaches the root."""
    parent = np.asarray(parent, dtype=np.int64)
    B1 = parent.shape[0]
    if B1 < 1 or parent[0] != -1:
        raise ValueError("parent[0] must be -1 (the main branch is the root)")
    depth = np.zeros(B1, dtype=np.int64)
    for i in range(1, B1):
        p = int(parent[i])
        if not 0 <= p < i:
            raise ValueError(f"parent[{i}] = {p} is not in [0, {i})")
        depth[i] = depth[p] + 1
    return depth


def root_path(parent, i: int) -> list[int]:
    """Branch indices from i up to the root, following parents."""
    path = [int(i)]
    while path[-1] != 0:
        path.append(int(parent[path[-1]]))
        if len(path) > len(parent):
            raise ValueError("parent chain does not reach the root")
    return path


def state_violations(state, parent, S_t: int) -> list[tuple[int, str]]:
    """[SF] introduction, Fig. 1-(b): a draft inherits its parent's state and
    unmasks at most S_t further positions.  Returns the offending drafts."""
    state = np.asarray(state)
    bad = []
    for i in range(1, state.shape[0]):
        p = int(parent[i])
        known = state[p] != MASK
        if np.any(state[i][known] != state[p][known]):
            bad.append((i, "changes or re-masks a parent position"))
            continue
        new = int(np.sum((state[p] == MASK) & (state[i] != MASK)))
        if new > S_t:
            bad.append((i, f"unmasks {new} > {S_t} positions"))
    return bad


# ----------------------------------------------------------------------------
# O3 — attention of every branch against [shared context | own block]
# ----------------------------------------------------------------------------


def _keys_for(k_blk, v_blk, k_ctx, v_ctx, i, g):
    K = np.concatenate([k_ctx[g], k_blk[i, :, g]], axis=0)
    V = np.concatenate([v_ctx[g], v_blk[i, :, g]], axis=0)
    return K, V


def attention(q, k_blk, v_blk, k_ctx, v_ctx, scale):
    """Full-softmax definition.  [SF] introduction and App. A.1: in-block
    attention is bidirectional and every output depends on every key of the
    shared prefix and of the branch's own block; no key is masked.  Query head
    h reads KV head h // (Hq/Hkv) (grouped-query attention, [SF] Sec. 3.3).

    q [B1][N][Hq][d], k_blk/v_blk [B1][N][Hkv][d], k_ctx/v_ctx [Hkv][L][d]
    (any float dtype; computed in fp64).  Returns o [B1][N][Hq][d] and the
    natural-log log-sum-exp lse = m + ln Z of the scaled scores [B1][N][Hq]."""
    q = np.asarray(q, np.float64)
    k_blk = np.asarray(k_blk, np.float64)
    v_blk = np.asarray(v_blk, np.float64)
    k_ctx = np.asarray(k_ctx, np.float64)
    v_ctx = np.asarray(v_ctx, np.float64)
    B1, N, Hq, d = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    o = np.empty((B1, N, Hq, d))
    lse = np.empty((B1, N, Hq))
    for i in range(B1):
        for h in range(Hq):
            K, V = _keys_for(k_blk, v_blk, k_ctx, v_ctx, i, h // G)
            s = (q[i, :, h, :] @ K.T) * scale          # [N][L+N]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            Z = e.sum(axis=1, keepdims=True)
            o[i, :, h, :] = (e @ V) / Z
            lse[i, :, h] = (m + np.log(Z))[:, 0]
    return o, lse


def attention_partial(qrows, K, V, scale):
    """Streaming-softmax state (m, Z, O) of rows against one key set, [SF]
    App. A.1 (per-row running maximum, denominator and normalised output)."""
    s = (qrows @ K.T) * scale
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    Z = e.sum(axis=1)
    O = (e @ V) / Z[:, None]
    return m, Z, O


def lse_merge(parts):
    """Merge (m, Z, O) states of disjoint key sets into the state of their
    union: m = max m_p, Z = sum Z_p e^(m_p - m), O = sum Z_p e^(m_p - m) O_p / Z."""
    m = np.max(np.stack([p[0] for p in parts]), axis=0)
    w = [p[1] * np.exp(p[0] - m) for p in parts]
    Z = np.sum(np.stack(w), axis=0)
    O = np.sum(np.stack([wi[:, None] * p[2] for wi, p in zip(w, parts)]), axis=0) / Z[:, None]
    return m, Z, O


def attention_split_merge(q, k_blk, v_blk, k_ctx, v_ctx, scale, ctx_splits=1):
    """The same attention computed as the hot path does: the context split into
    ctx_splits key ranges, the branch's own block as one more, states merged by
    log-sum-exp.  Tested equal to attention()."""
    q = np.asarray(q, np.float64)
    k_blk = np.asarray(k_blk, np.float64)
    v_blk = np.asarray(v_blk, np.float64)
    k_ctx = np.asarray(k_ctx, np.float64)
    v_ctx = np.asarray(v_ctx, np.float64)
    B1, N, Hq, d = q.shape
    Hkv = k_blk.shape[2]
    L = k_ctx.shape[1]
    G = Hq // Hkv
    bounds = np.linspace(0, L, ctx_splits + 1).astype(int)
    o = np.empty((B1, N, Hq, d))
    lse = np.empty((B1, N, Hq))
    for i in range(B1):
        for h in range(Hq):
            g = h // G
            parts = []
            for a, b in zip(bounds[:-1], bounds[1:]):
                if b > a:
                    parts.append(attention_partial(q[i, :, h], k_ctx[g, a:b], v_ctx[g, a:b], scale))
            parts.append(attention_partial(q[i, :, h], k_blk[i, :, g], v_blk[i, :, g], scale))
            m, Z, O = lse_merge(parts)
            o[i, :, h] = O
            lse[i, :, h] = m + np.log(Z)
    return o, lse


# ----------------------------------------------------------------------------
# O4, O5 — masked rows and the LM head
# ----------------------------------------------------------------------------


def masked_rows(state) -> np.ndarray:
    """Flat row ids i*N + n of every masked position, in (i, n) order.  [SF]
    introduction: the forward map returns distributions for the masked
    positions of the active block."""
    state = np.asarray(state)
    B1, N = state.shape
    out = [i * N + n for i in range(B1) for n in range(N) if state[i, n] == MASK]
    return np.asarray(out, dtype=np.int64)


def lm_head(hidden, rows, w, v_chunk=8192):
    """logits[r][v] = sum_k hidden[rows[r]][k] * w[v][k], in fp64.  [SF]
    Appendix B: the language-model head is a plain dense product."""
    h = np.asarray(hidden, np.float64)[np.asarray(rows, np.int64)]
    V = w.shape[0]
    out = np.empty((h.shape[0], V))
    for a in range(0, V, v_chunk):
        b = min(V, a + v_chunk)
        out[:, a:b] = h @ np.asarray(w[a:b], np.float64).T
    return out


# ----------------------------------------------------------------------------
# O6 — counter-based noise, Gumbel-max token, max-softmax confidence
# ----------------------------------------------------------------------------
# Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy
# as 1, 2, 3", SC'11): ten rounds of two 64x64->128 multiplies, key bumped by
# Weyl constants between rounds.
_PH_M0 = np.uint64(0xD2E7470EE14C6C93)
_PH_M1 = np.uint64(0xCA5A826395121157)
_PH_W0 = np.uint64(0x9E3779B97F4A7C15)
_PH_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a: np.ndarray, b: np.uint64):
    a_lo, a_hi = a & _LO32, a >> _S32
    b_lo, b_hi = b & _LO32, b >> _S32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> _S32) + (lh & _LO32) + (hl & _LO32)
    lo = (ll & _LO32) | ((mid & _LO32) << _S32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds.  ctr: uint64 [..., 4]; key: uint64 [..., 2]
    (broadcast).  Returns uint64 [..., 4]."""
    with np.errstate(over="ignore"):
        c = np.asarray(ctr, dtype=np.uint64)
        k = np.asarray(key, dtype=np.uint64)
        c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
        k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
        k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
        for r in range(10):
            if r:
                k0 = k0 + _PH_W0
                k1 = k1 + _PH_W1
            hi0, lo0 = _mulhilo64(c0, _PH_M0)
            hi1, lo1 = _mulhilo64(c2, _PH_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        return np.stack([c0, c1, c2, c3], axis=-1)


def noise_words(seed: int, step: int, pos: int, v, stream: int = 0) -> np.ndarray:
    """32-bit noise word for (seed, step, position, vocab id).

    Counter-based hash (SPOT, coupled-noise match: target and drafter share
    per-position Gumbel noise).  Key = (seed, 0); counter = (v >> 3, position,
    step, stream), all as unsigned 64-bit; output word (v & 7) >> 1 of the
    four, low half for even v and high half for odd v.  Stream 0 is the
    commit's noise; other streams are independent draws for other uses."""
    v = np.asarray(v, dtype=np.int64)
    m64 = (1 << 64) - 1
    blocks, which = np.unique(v >> 3, return_inverse=True)   # one call per 8 ids
    ctr = np.zeros((blocks.shape[0], 4), dtype=np.uint64)
    ctr[:, 0] = blocks.astype(np.uint64)
    ctr[:, 1] = np.uint64(int(pos) & m64)
    ctr[:, 2] = np.uint64(int(step) & m64)
    ctr[:, 3] = np.uint64(int(stream) & m64)
    key = np.array([int(seed) & m64, 0], dtype=np.uint64)
    out = philox4x64_10(ctr, key)
    word = out[which.reshape(v.shape), (v & 7) >> 1]
    half = (v & 1).astype(np.uint64) * np.uint64(32)
    return ((word >> half) & _LO32).astype(np.uint32)


def gumbel_from_words(w) -> np.ndarray:
    """Standard Gumbel(0, 1) by inversion: u = (w + 1/2) 2^-32 in (0, 1),
    g = fl32(-ln(-ln u)) with both logarithms in fp64."""
    u = (np.asarray(w, dtype=np.float64) + 0.5) * 2.0 ** -32
    return (-np.log(-np.log(u))).astype(np.float32)


def gumbel(seed: int, step: int, pos: int, v) -> np.ndarray:
    return gumbel_from_words(noise_words(seed, step, pos, v))


def first_argmax(x) -> int:
    """Lowest index attaining the maximum."""
    x = np.asarray(x)
    return int(np.flatnonzero(x == x.max())[0])


def sample_token(logits_row, T: float, seed: int, step: int, pos: int, g=None) -> int:
    """Token of one masked row from fp32 logits.

    T = 0: greedy, the lowest vocab id attaining max logit.  T > 0: Gumbel-max
    with invT = fl32(1/T), key_v = fl32(fl32(l_v * invT) + g_v), the lowest
    vocab id attaining max key (SPOT, coupled-noise match and Prop. 2: given
    the noise the transition is deterministic).  g, if given, is the noise row
    gumbel(seed, step, pos, 0..V-1) already drawn."""
    lr = np.asarray(logits_row, dtype=np.float32)
    if T == 0.0:
        return first_argmax(lr)
    inv_t = np.float32(1.0) / np.float32(T)
    if g is None:
        g = gumbel(seed, step, pos, np.arange(lr.shape[0]))
    key = (lr * inv_t).astype(np.float32) + g
    return first_argmax(key.astype(np.float32))


def confidence_sum(logits_row) -> float:
    """S = sum_v exp(l_v - l_max) in fp64 from the fp32 logits; the max-softmax
    confidence is 1/S (unscaled logits, independent of T)."""
    lr = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    return float(np.sum(np.exp(lr - lr.max())))


# ----------------------------------------------------------------------------
# O7 — confidence-based unmasking
# ----------------------------------------------------------------------------


def commit(logits, rows, state, parent, T, seed, step0, pos0, k_max=1, tau=0.0):
    """One commit of every branch from its fp32 logits.

    [SF] introduction: an unmasking rule selects high-confidence masked
    positions; [SPOT] "Important context": exact decoding commits one position
    per forward, the one the target commits next.  Per branch i: each masked
    position n gets token tok(i, n) drawn with noise keyed by step
    step0 + depth(i) and position pos0 + n; positions are ranked by S
    ascending (confidence descending), ties to the lower n; the first is
    committed, and while fewer than k_max are taken, further positions with
    fl32(1/S) >= tau.

    Returns next_state [B1][N], commit_pos [B1][k_max] (-1 padded),
    token [M], conf [M] (fp32) and S [M] (fp64)."""
    logits = np.asarray(logits, dtype=np.float32)
    state = np.asarray(state)
    B1, N = state.shape
    rows = np.asarray(rows, dtype=np.int64)
    depth = tree_depths(parent)
    M = rows.shape[0]
    token = np.empty(M, dtype=np.int32)
    S = np.empty(M, dtype=np.float64)
    noise = {}   # rows with the same (step, position) draw the same noise
    for r in range(M):
        i, n = divmod(int(rows[r]), N)
        step, pos = step0 + int(depth[i]), pos0 + n
        g = None
        if T != 0.0:
            if (step, pos) not in noise:
                noise[(step, pos)] = gumbel(seed, step, pos, np.arange(logits.shape[1]))
            g = noise[(step, pos)]
        token[r] = sample_token(logits[r], T, seed, step, pos, g)
        S[r] = confidence_sum(logits[r])
    conf = (1.0 / S).astype(np.float32)
    where = {int(rows[r]): r for r in range(M)}
    next_state = state.copy()
    commit_pos = np.full((B1, k_max), -1, dtype=np.int32)
    for i in range(B1):
        cand = [(S[where[i * N + n]], n) for n in range(N) if state[i, n] == MASK]
        if not cand:
            continue
        cand.sort()
        taken = []
        for s_val, n in cand:
            if not taken:
                taken.append(n)
            elif len(taken) < k_max and np.float32(1.0 / s_val) >= np.float32(tau):
                taken.append(n)
            else:
                break
        for j, n in enumerate(taken):
            commit_pos[i, j] = n
            next_state[i, n] = token[where[i * N + n]]
    return next_state, commit_pos, token, conf, S


# ----------------------------------------------------------------------------
# O8 — state-equality walk over the draft tree
# ----------------------------------------------------------------------------


def match_tree(state, next_state, commit_pos, parent, S_max=-1):
    """Longest run of drafted states the target itself produces.

    [SF] introduction: a later main-branch state that equals a cached draft
    reuses that draft's logits; [SPOT] "How does SPOT draft and verify?":
    accept the longest prefix consistent with the target's own trajectory.
    From the main branch, repeatedly find the lowest draft index, one tree
    level below the current branch, whose state equals the current branch's
    committed next state, and move there.  Stops on a miss, when the current
    branch had nothing to commit, or after B hops.

    The level condition: a draft at depth d stands for the trajectory's state
    after d steps, and its own commit draws the noise of step step0 + d.  A
    draft at another depth holding the right state would commit with another
    step's noise, and the accepted run would leave the draft-free trajectory
    ([SPOT] "Is the output exact when the target samples?", Proposition 2).

    With S_max >= 0 the drafts are first checked to extend their parent by at
    most S_max positions; a violation returns status SFV_E_STATE and accepts
    nothing.  Returns (chain [B1] -1 padded, h, status)."""
    state = np.asarray(state)
    next_state = np.asarray(next_state)
    commit_pos = np.asarray(commit_pos).reshape(state.shape[0], -1)
    B1 = state.shape[0]
    chain = np.full(B1, -1, dtype=np.int32)
    if S_max >= 0 and state_violations(state, parent, S_max):
        return chain, 0, SFV_E_STATE
    depth = tree_depths(parent)
    cur, h = 0, 0
    while h < B1 - 1:
        if commit_pos[cur, 0] == -1:
            break
        hit = [j for j in range(1, B1)
               if depth[j] == depth[cur] + 1 and np.array_equal(state[j], next_state[cur])]
        if not hit:
            break
        cur = hit[0]
        chain[h] = cur
        h += 1
    return chain, h, SFV_OK


def final_state(next_state, chain, h):
    """The block state after accepting h drafted transitions plus the target's
    own commit on the last accepted state."""
    return np.asarray(next_state)[0 if h == 0 else int(chain[h - 1])].copy()


# ----------------------------------------------------------------------------
# whole step (used for the CPU baseline timing)
# ----------------------------------------------------------------------------


def verify_step(q, k_blk, v_blk, k_ctx, v_ctx, hidden, w, state, parent, T, seed,
                step0, pos0, scale, S_max=-1):
    o, lse = attention(q, k_blk, v_blk, k_ctx, v_ctx, scale)
    rows = masked_rows(state)
    logits = lm_head(hidden, rows, w).astype(np.float32)
    nxt, cpos, tok, conf, S = commit(logits, rows, state, parent, T, seed, step0, pos0)
    chain, h, status = match_tree(state, nxt, cpos, parent, S_max)
    return dict(o=o, lse=lse, rows=rows, logits=logits, next_state=nxt, commit_pos=cpos,
                token=tok, conf=conf, chain=chain, h=h, status=status)
