"""Pins of the rejection-sampling verification oracle (D3D explainer: lossless
verification of drafted blocks with the proposal probabilities)."""
import numpy as np
import pytest
from scipy import stats

from oracle import oracle as O
from oracle import reject as R


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _case(rng, B, V, T, drift):
    logits = (rng.standard_normal((B + 1, V)) * 1.5).astype(np.float32)
    q = np.stack([_softmax((logits[t] / T + drift * rng.standard_normal(V))) for t in range(B)]).astype(np.float32)
    return logits, q


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_first_emitted_token_is_distributed_as_p(T):
    """Over many seeds the first token the rule emits (x_0 when accepted, else
    the residual draw) follows p_0, whatever q is: the rule is lossless."""
    rng = np.random.default_rng(1)
    V, B = 6, 1
    logits, q = _case(rng, B, V, T, drift=1.2)
    p0 = R.target_probs(logits[0], T)
    counts = np.zeros(V)
    n = 6000
    drng = np.random.default_rng(2)
    for s in range(n):
        x = int(drng.choice(V, p=q[0] / q[0].sum()))
        a, c = R.verify_tray(logits, q, [x], T, seed=s, step=3, pos0=10)
        counts[x if a == 1 else c] += 1
    chi = stats.chisquare(counts, n * p0)
    assert chi.pvalue > 1e-3, (counts / n, p0)


def test_first_two_tokens_follow_the_target():
    """With logits independent of the tokens, the first two emitted tokens
    follow p_0 x p_1."""
    rng = np.random.default_rng(3)
    V, B, T = 4, 2, 1.0
    logits, q = _case(rng, B, V, T, drift=1.0)
    p0, p1 = R.target_probs(logits[0], T), R.target_probs(logits[1], T)
    counts = np.zeros((V, V))
    n = 8000
    drng = np.random.default_rng(4)
    got = 0
    for s in range(n):
        x = [int(drng.choice(V, p=q[t] / q[t].sum())) for t in range(B)]
        a, c = R.verify_tray(logits, q, x, T, seed=100 + s, step=0, pos0=0)
        if a == 0:
            continue  # the second emitted token would need a new target pass
        first = x[0]
        second = x[1] if a == 2 else c
        counts[first, second] += 1
        got += 1
    # conditional on the first being accepted (a >= 1), the second follows p1
    marg = counts.sum(axis=0)
    chi = stats.chisquare(marg, marg.sum() * p1)
    assert chi.pvalue > 1e-3


def test_equal_proposal_accepts_everything():
    rng = np.random.default_rng(5)
    V, B, T = 50, 8, 1.0
    logits = (rng.standard_normal((B + 1, V))).astype(np.float32)
    q = np.stack([R.target_probs(logits[t], T) for t in range(B)]).astype(np.float32)
    for s in range(20):
        x = [int(np.argmax(q[t] + rng.random(V) * 1e-9)) for t in range(B)]
        q2 = q.astype(np.float64).copy()
        for t in range(B):
            q2[t] = R.target_probs(logits[t], T)
        a, c = R.verify_tray(logits, q2.astype(np.float32) * np.float32(0.999999), x, T, seed=s, step=1, pos0=0)
        assert a == B


def test_greedy_is_the_argmax_check():
    rng = np.random.default_rng(6)
    V, B = 30, 5
    logits = rng.standard_normal((B + 1, V)).astype(np.float32)
    q = np.full((B, V), 1.0 / V, np.float32)
    best = [O.first_argmax(logits[t]) for t in range(B + 1)]
    x = list(best[:B])
    x[3] = (best[3] + 1) % V
    a, c = R.verify_tray(logits, q, x, 0.0, 1, 1, 0)
    assert a == 3 and c == best[3]
    a, c = R.verify_tray(logits, q, best[:B], 0.0, 1, 1, 0)
    assert a == B and c == best[B]


def test_rejections_emit_residual_support_only():
    rng = np.random.default_rng(7)
    V, B, T = 12, 3, 1.0
    for s in range(200):
        logits, q = _case(rng, B, V, T, drift=2.0)
        x = [int(np.argmax(q[t])) for t in range(B)]
        a, c = R.verify_tray(logits, q, x, T, seed=s, step=2, pos0=5)
        if a < B:
            p = R.target_probs(logits[a], T)
            assert p[c] > q[a, c]


def test_match_tray():
    k = [1, 1, 2, 2, 16, 1]
    alt = [5, 7, 5, 9, 3, 7]
    assert R.match_tray(1, 7, k, alt) == 1
    assert R.match_tray(2, 9, k, alt) == 3
    assert R.match_tray(16, 3, k, alt) == 4
    assert R.match_tray(2, 6, k, alt) == -1


def test_noise_streams_are_independent():
    a = O.noise_words(1, 2, 3, np.arange(64), stream=0)
    b = O.noise_words(1, 2, 3, np.arange(64), stream=1)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, O.noise_words(1, 2, 3, np.arange(64)))


def _qkv(rng, B1, N, L, Hq, Hkv, d):
    f = lambda *s: rng.standard_normal(s)
    return f(B1, N, Hq, d), f(B1, N, Hkv, d), f(B1, N, Hkv, d), f(Hkv, L, d), f(Hkv, L, d)


def test_tray_attention_against_torch_masked_sdpa():
    import torch
    rng = np.random.default_rng(11)
    B1, N, L, Hq, Hkv, d = 3, 5, 7, 4, 2, 8
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    o, lse = R.tray_attention(q, kb, vb, kc, vc, 0.4)
    G = Hq // Hkv
    mask = torch.ones(N, L + N, dtype=torch.bool)
    mask[:, L:] = torch.tril(torch.ones(N, N, dtype=torch.bool))
    for i in range(B1):
        for h in range(Hq):
            g = h // G
            K = torch.from_numpy(np.concatenate([kc[g], kb[i, :, g]]))
            V = torch.from_numpy(np.concatenate([vc[g], vb[i, :, g]]))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[i, :, h])[None], K[None], V[None], attn_mask=mask[None], scale=0.4)[0]
            np.testing.assert_allclose(o[i, :, h], ref.numpy(), atol=1e-12)


def test_tray_attention_last_position_sees_the_whole_tray():
    rng = np.random.default_rng(12)
    B1, N, L, Hq, Hkv, d = 2, 6, 9, 2, 1, 8
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    o, lse = R.tray_attention(q, kb, vb, kc, vc, 0.3)
    o2, lse2 = O.attention(q, kb, vb, kc, vc, 0.3)
    np.testing.assert_allclose(o[:, -1], o2[:, -1], atol=1e-12)
    np.testing.assert_allclose(lse[:, -1], lse2[:, -1], rtol=1e-13)
    # position 0 sees the context and itself only
    o0, _ = O.attention(q[:, :1], kb[:, :1], vb[:, :1], kc, vc, 0.3)
    np.testing.assert_allclose(o[:, 0], o0[:, 0], atol=1e-12)
