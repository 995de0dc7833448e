"""Pins of the oracle attention (O3): the full-softmax definition against the
split-context + block + log-sum-exp merge form (brute force), closed forms,
and torch's CPU scaled_dot_product_attention in fp64 as a library routine.

SpecFold, App. A.1 and Sec. 3.3: streaming (m, Z, O) state over the
concatenated prefix and block keys, bidirectional, grouped-query heads."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def _rand(rng, B1=3, N=8, L=64, Hq=4, Hkv=2, d=32):
    q = rng.standard_normal((B1, N, Hq, d))
    kb = rng.standard_normal((B1, N, Hkv, d))
    vb = rng.standard_normal((B1, N, Hkv, d))
    kc = rng.standard_normal((Hkv, L, d))
    vc = rng.standard_normal((Hkv, L, d))
    return q, kb, vb, kc, vc


@pytest.mark.parametrize("shape", [dict(), dict(B1=2, N=5, L=7, Hq=8, Hkv=1, d=16),
                                   dict(B1=4, N=3, L=0, Hq=2, Hkv=2, d=8),
                                   dict(B1=1, N=1, L=33, Hq=8, Hkv=8, d=4)])
@pytest.mark.parametrize("splits", [1, 3])
def test_split_merge_equals_full(shape, splits):
    rng = np.random.default_rng(7)
    args = _rand(rng, **shape)
    scale = 1 / np.sqrt(args[0].shape[-1])
    o1, l1 = O.attention(*args, scale)
    o2, l2 = O.attention_split_merge(*args, scale, ctx_splits=splits)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


def test_equal_keys_closed_form():
    rng = np.random.default_rng(1)
    B1, N, L, Hq, Hkv, d = 2, 4, 10, 4, 2, 8
    q = rng.standard_normal((B1, N, Hq, d))
    k = rng.standard_normal(d)
    kb = np.broadcast_to(k, (B1, N, Hkv, d)).copy()
    kc = np.broadcast_to(k, (Hkv, L, d)).copy()
    vb = rng.standard_normal((B1, N, Hkv, d))
    vc = rng.standard_normal((Hkv, L, d))
    o, lse = O.attention(q, kb, vb, kc, vc, 0.5)
    for i in range(B1):
        for h in range(Hq):
            g = h // 2
            s = 0.5 * q[i, :, h] @ k
            np.testing.assert_allclose(lse[i, :, h], s + np.log(L + N), rtol=0, atol=1e-12)
            mean_v = np.concatenate([vc[g], vb[i, :, g]]).mean(axis=0)
            np.testing.assert_allclose(o[i, :, h], np.broadcast_to(mean_v, (N, d)), atol=1e-12)


def test_single_key_closed_form():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 1, 2, 4))
    kb = rng.standard_normal((2, 1, 1, 4))
    vb = rng.standard_normal((2, 1, 1, 4))
    kc = np.zeros((1, 0, 4)); vc = np.zeros((1, 0, 4))
    o, lse = O.attention(q, kb, vb, kc, vc, 0.3)
    for i in range(2):
        for h in range(2):
            np.testing.assert_allclose(o[i, 0, h], vb[i, 0, 0], atol=1e-15)
            np.testing.assert_allclose(lse[i, 0, h], 0.3 * q[i, 0, h] @ kb[i, 0, 0], atol=1e-14)


def test_against_torch_sdpa_fp64():
    rng = np.random.default_rng(3)
    B1, N, L, Hq, Hkv, d = 3, 8, 64, 4, 2, 32
    q, kb, vb, kc, vc = _rand(rng, B1, N, L, Hq, Hkv, d)
    scale = 1 / np.sqrt(d)
    o, lse = O.attention(q, kb, vb, kc, vc, scale)
    G = Hq // Hkv
    for i in range(B1):
        K = np.concatenate([kc, kb[i].transpose(1, 0, 2)], axis=1)      # [Hkv][L+N][d]
        Vv = np.concatenate([vc, vb[i].transpose(1, 0, 2)], axis=1)
        K = np.repeat(K, G, axis=0)                                    # heads h -> h // G
        Vv = np.repeat(Vv, G, axis=0)
        Q = q[i].transpose(1, 0, 2)                                    # [Hq][N][d]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(Vv), scale=scale).numpy()
        np.testing.assert_allclose(o[i].transpose(1, 0, 2), ref, atol=1e-12)
        s = torch.from_numpy(Q) @ torch.from_numpy(K).transpose(-1, -2) * scale
        ref_lse = torch.logsumexp(s, dim=-1).numpy()                   # [Hq][N]
        np.testing.assert_allclose(lse[i].T, ref_lse, atol=1e-12)


def test_gqa_mapping_detects_wrong_head():
    # a plausible mistake (kv head h % Hkv instead of h // G) changes the output
    rng = np.random.default_rng(4)
    q, kb, vb, kc, vc = _rand(rng, 1, 4, 8, 4, 2, 8)
    o, _ = O.attention(q, kb, vb, kc, vc, 0.35)
    q_swapped = q[:, :, [0, 2, 1, 3]]
    o2, _ = O.attention(q_swapped, kb, vb, kc, vc, 0.35)
    assert np.max(np.abs(o2[:, :, [0, 2, 1, 3]] - o)) > 1e-3


def test_block_keys_are_bidirectional():
    # every block key reaches every block query: permuting block keys/values
    # together leaves outputs unchanged; dropping the last key changes row 0
    rng = np.random.default_rng(5)
    q, kb, vb, kc, vc = _rand(rng, 1, 6, 5, 2, 1, 8)
    o, lse = O.attention(q, kb, vb, kc, vc, 0.4)
    perm = rng.permutation(6)
    o2, lse2 = O.attention(q, kb[:, perm], vb[:, perm], kc, vc, 0.4)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    _, lse3 = O.attention(q[:, :1], kb[:, :5], vb[:, :5], kc, vc, 0.4)
    assert np.all(np.abs(lse3[0, 0] - lse[0, 0]) > 1e-6)
