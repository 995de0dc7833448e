"""CPU oracle for verifying drafted blocks of an autoregressive target by
rejection sampling, and for serving the prepared tray that matches.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

[D3D] the diffusion-drafter explainer ("D3D diffusion drafter -- Asynchronous
speculative decoding"): the target verifies a drafted block by rejection
sampling with the proposal probabilities, the standard rule that keeps the
target's distribution; the drafter prepares one tray per plausible outcome
(the tokens accepted before a rejection point, another token at that point,
a fresh block after it, plus one tray for the case that every token passes),
and the tray matching the verified prefix is served (a cache hit), else the
target waits for a fresh draft (a miss).

Readings (the page states the rule but not its arithmetic):
  * Target distribution at a verified position: p = softmax(fl32(l * invT))
    in fp64 from fp32 logits l, invT = fl32(1/T).  T = 0 is greedy.
  * Drafted token x with proposal probability q(x) (fp32) is accepted iff
    u * q(x) < p(x), with u = (w + 1/2) 2^-32 from noise stream 1 at
    (seed, step0 + tray, pos0 + t): the usual min(1, p/q) test.
  * The first rejected position a emits a token from the residual
    max(0, p - q) normalised: the Gumbel-max argmax_v ln(p_v - q_v) + g_v over
    v with p_v > q_v, g in fp64 from noise stream 2 at position pos0 + a.  If
    all B pass, the bonus token is argmax_v fl32(l_v invT) + g_v (stream 2,
    position pos0 + B).  Ties go to the lower id.  An empty residual (p <= q
    everywhere, possible only by rounding) emits the first argmax of
    fl32(l invT).
  * T = 0: x is accepted iff it is the first argmax of l; the emitted token is
    the first argmax at position a (or B).
  * The served tray is the lowest-indexed tray whose (rejection point,
    token there) equals the verified (accepted count, emitted token); none
    matching is a miss (-1).

Pins (tests/test_oracle_reject.py): the first emitted token is distributed as
p (chi-square over seeds, the losslessness of the rule); the first two
emitted tokens are distributed as p_0 x p_1; q = p accepts everything; T = 0
is the greedy check; rejections emit only tokens with p > q.
"""
from __future__ import annotations

import numpy as np

from .oracle import first_argmax, noise_words

STREAM_ACCEPT = 1
STREAM_SAMPLE = 2


def scaled_logits(logits_row, T: float) -> np.ndarray:
    """fl32(l * fl32(1/T)) as fp64."""
    lr = np.asarray(logits_row, dtype=np.float32)
    inv_t = np.float32(1.0) / np.float32(T)
    return (lr * inv_t).astype(np.float32).astype(np.float64)


def target_probs(logits_row, T: float) -> np.ndarray:
    z = scaled_logits(logits_row, T)
    e = np.exp(z - z.max())
    return e / e.sum()


def uniform(seed: int, step: int, pos: int) -> float:
    w = noise_words(seed, step, pos, np.array([0]), stream=STREAM_ACCEPT)[0]
    return (float(w) + 0.5) * 2.0 ** -32


def gumbel64(seed: int, step: int, pos: int, v) -> np.ndarray:
    w = noise_words(seed, step, pos, v, stream=STREAM_SAMPLE)
    u = (w.astype(np.float64) + 0.5) * 2.0 ** -32
    return -np.log(-np.log(u))


def _argmax_first(keys, valid=None) -> int:
    keys = np.asarray(keys, dtype=np.float64)
    if valid is not None:
        keys = np.where(valid, keys, -np.inf)
    return first_argmax(keys)


def verify_tray(logits, q, tokens, T: float, seed: int, step: int, pos0: int):
    """One drafted block: logits [B+1][V] fp32 (the target's distributions at
    the B drafted positions and the bonus position), q [B][V] fp32, tokens
    [B].  Returns (accepted count a, emitted token)."""
    logits = np.asarray(logits, dtype=np.float32)
    q = np.asarray(q, dtype=np.float32)
    B = len(tokens)
    a = B
    for t in range(B):
        x = int(tokens[t])
        if T == 0.0:
            ok = x == first_argmax(logits[t])
        else:
            p = target_probs(logits[t], T)
            ok = uniform(seed, step, pos0 + t) * float(q[t, x]) < p[x]
        if not ok:
            a = t
            break
    V = logits.shape[1]
    if T == 0.0:
        return a, first_argmax(logits[a])
    g = gumbel64(seed, step, pos0 + a, np.arange(V))
    if a < B:
        r = target_probs(logits[a], T) - q[a].astype(np.float64)
        pos = r > 0
        if not pos.any():  # p <= q everywhere, possible only by rounding
            return a, first_argmax(scaled_logits(logits[a], T))
        keys = np.where(pos, np.log(np.where(pos, r, 1.0)) + g, -np.inf)
        return a, _argmax_first(keys, pos)
    return a, _argmax_first(scaled_logits(logits[B], T) + g)


def verify_trays(logits, q, tokens, T: float, seed: int, step0: int, pos0: int):
    """Every tray j (noise step step0 + j).  logits [n_trays][B+1][V],
    q [n_trays][B][V], tokens [n_trays][B] -> (n_accept, next_token)."""
    out_a, out_c = [], []
    for j in range(len(tokens)):
        a, c = verify_tray(logits[j], q[j], tokens[j], T, seed, step0 + j, pos0)
        out_a.append(a)
        out_c.append(c)
    return np.array(out_a, dtype=np.int64), np.array(out_c, dtype=np.int64)


def match_tray(accepted: int, token: int, tray_k, tray_alt) -> int:
    """Lowest tray whose (rejection point, token there) is the verified
    (accepted count, emitted token); -1 on a miss."""
    for j in range(len(tray_k)):
        if int(tray_k[j]) == accepted and int(tray_alt[j]) == token:
            return j
    return -1


def tray_attention(q, k_blk, v_blk, k_ctx, v_ctx, scale):
    """Attention of an autoregressive target over drafted trays ([D3D] the
    target verifies the prepared trays in one packed pass): each tray i
    continues the shared context, so position n of tray i attends the L
    context keys and the tray's block keys 0..n.  Shapes as oracle.attention;
    fp64.  Returns o [B1][N][Hq][d], lse [B1][N][Hq] (natural log)."""
    q = np.asarray(q, np.float64)
    k_blk = np.asarray(k_blk, np.float64)
    v_blk = np.asarray(v_blk, np.float64)
    k_ctx = np.asarray(k_ctx, np.float64)
    v_ctx = np.asarray(v_ctx, np.float64)
    B1, N, Hq, d = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    L = k_ctx.shape[1]
    o = np.empty((B1, N, Hq, d))
    lse = np.empty((B1, N, Hq))
    for i in range(B1):
        for h in range(Hq):
            g = h // G
            K = np.concatenate([k_ctx[g], k_blk[i, :, g]], axis=0)
            V = np.concatenate([v_ctx[g], v_blk[i, :, g]], axis=0)
            s = (q[i, :, h, :] @ K.T) * scale                  # [N][L+N]
            visible = np.ones_like(s, dtype=bool)
            visible[:, L:] = np.tril(np.ones((N, N), dtype=bool))
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            Z = e.sum(axis=1, keepdims=True)
            o[i, :, h, :] = (e @ V) / Z
            lse[i, :, h] = (m + np.log(Z))[:, 0]
    return o, lse
