"""Pins of the folded-verification oracle (SpecFold Sec. 3.2, App. A-B)."""
import json
import os

import numpy as np
import pytest

from branch_verify_amd import synth
from oracle import fold as F
from oracle import oracle as O

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_gate_hand_worked_fixture():
    with open(os.path.join(HERE, "fold_gate_tiny.json")) as fh:
        fx = json.load(fh)
    H = np.array(fx["H"], dtype=np.float64)
    parent = np.array(fx["parent"])
    for case in fx["cases"]:
        rec, src, rows, off = F.fold_gate(H, parent, case["delta"])
        assert rec.astype(int).tolist() == case["recompute"], case["delta"]
        assert src.tolist() == case["src"], case["delta"]
        assert rows.tolist() == case["rec_rows"], case["delta"]
        assert off.tolist() == case["branch_off"], case["delta"]


def _tree(rng, B1, kind):
    if kind == "chain":
        return np.array([-1] + list(range(B1 - 1)))
    if kind == "star":
        return np.array([-1] + [0] * (B1 - 1))
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, B1)])


@pytest.mark.parametrize("kind", ["chain", "star", "random"])
def test_sources_are_nearest_recomputed_ancestor(kind):
    """Brute force: walk each root path and take the first branch in which the
    position is recomputed; the compacted lists are the flags in order."""
    rng = np.random.default_rng(3)
    B1, N, D = 12, 9, 16
    parent = _tree(rng, B1, kind)
    H = rng.standard_normal((B1, N, D))
    for i in range(1, B1):  # children close to their parents at some positions
        near = rng.random(N) < 0.6
        H[i, near] = H[parent[i], near] + 0.01 * rng.standard_normal((int(near.sum()), D))
    rec, src, rows, off = F.fold_gate(H, parent, 0.1)
    assert rec[0].all()
    for i in range(B1):
        for n in range(N):
            want = next(b for b in O.root_path(parent, i) if rec[b, n])
            assert src[i, n] == want
    flat = [i * N + n for i in range(B1) for n in range(N) if rec[i, n]]
    assert rows.tolist() == flat
    for i in range(B1):
        seg = rows[off[i]:off[i + 1]]
        assert np.all(seg // N == i) and seg.size == rec[i].sum()


def test_gate_matches_relative_residual():
    """num <= delta^2 den is rho <= delta away from the boundary; rho from
    numpy.linalg.norm."""
    rng = np.random.default_rng(4)
    B1, N, D = 6, 16, 64
    parent = _tree(rng, B1, "random")
    H = rng.standard_normal((B1, N, D))
    for i in range(1, B1):
        H[i] = H[parent[i]] + rng.uniform(0, 0.3, (N, 1)) * rng.standard_normal((N, D))
    rec, *_ = F.fold_gate(H, parent, 0.1)
    for i in range(1, B1):
        for n in range(N):
            rho = np.linalg.norm(H[i, n] - H[parent[i], n]) / np.linalg.norm(H[parent[i], n])
            if abs(rho - 0.1) > 1e-9:
                assert rec[i, n] == (rho > np.float32(0.1))


def _qkv(rng, B1, N, L, Hq, Hkv, d):
    f = lambda *s: rng.standard_normal(s)
    return f(B1, N, Hq, d), f(B1, N, Hkv, d), f(B1, N, Hkv, d), f(Hkv, L, d), f(Hkv, L, d)


def test_nothing_folds_is_dense_attention():
    rng = np.random.default_rng(5)
    B1, N, L, Hq, Hkv, d = 4, 6, 10, 4, 2, 8
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    H = rng.standard_normal((B1, N, 16))
    rec, src, *_ = F.fold_gate(H, np.array([-1, 0, 1, 1]), -1.0)
    assert rec.all() and np.all(src == np.arange(B1)[:, None])
    o, lse = F.attention_folded(q, kb, vb, kc, vc, src, 0.3)
    o_d, lse_d = O.attention(q, kb, vb, kc, vc, 0.3)
    assert np.array_equal(o, o_d) and np.array_equal(lse, lse_d)


def test_everything_folds_copies_the_main_branch():
    """delta = inf folds every draft slot into the main branch: every branch
    then holds the main branch's tables and outputs."""
    rng = np.random.default_rng(6)
    B1, N, L, Hq, Hkv, d = 5, 4, 7, 2, 1, 8
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    H = rng.standard_normal((B1, N, 16))
    rec, src, rows, off = F.fold_gate(H, np.array([-1, 0, 0, 2, 3]), np.inf)
    assert rec[0].all() and not rec[1:].any() and np.all(src == 0)
    assert rows.tolist() == list(range(N)) and off.tolist() == [0] + [N] * B1
    o, lse = F.attention_folded(q, kb, vb, kc, vc, src, 0.25)
    o0, lse0 = O.attention(q[:1], kb[:1], vb[:1], kc, vc, 0.25)
    for i in range(B1):
        np.testing.assert_array_equal(o[i], o0[0])
        np.testing.assert_array_equal(lse[i], lse0[0])


@pytest.mark.parametrize("kind,delta", [("chain", 0.1), ("random", 0.1), ("star", 0.3), ("chain", 0.5)])
def test_chain_correction_equals_definition(kind, delta):
    """The hop-by-hop (m, Z, O) correction of the method reproduces the full
    attention over the branch's resolved table (fp64, up to rounding)."""
    rng = np.random.default_rng({"chain": 1, "random": 2, "star": 3}[kind] * 100 + int(delta * 10))
    B1, N, L, Hq, Hkv, d, D = 7, 6, 9, 4, 2, 8, 24
    parent = _tree(rng, B1, kind)
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    H = rng.standard_normal((B1, N, D))
    for i in range(1, B1):
        H[i] = H[parent[i]] + rng.uniform(0, 0.6, (N, 1)) * rng.standard_normal((N, D))
    rec, src, *_ = F.fold_gate(H, parent, delta)
    assert 0 < (~rec).sum() < rec[1:].size   # a mix of folded and recomputed slots
    o, lse = F.attention_folded(q, kb, vb, kc, vc, src, 0.35)
    o2, lse2 = F.attention_fold_chain(q, kb, vb, kc, vc, parent, rec, src, 0.35)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12)


def test_unresolved_keys_change_the_result():
    """A plausible mistake -- a folded query attending the branch's raw block
    table instead of its resolved one -- changes the outputs, so the pins
    above see whether keys are inherited."""
    rng = np.random.default_rng(8)
    B1, N, L, Hq, Hkv, d, D = 4, 5, 6, 2, 1, 8, 16
    parent = np.array([-1, 0, 1, 2])
    q, kb, vb, kc, vc = _qkv(rng, B1, N, L, Hq, Hkv, d)
    H = rng.standard_normal((B1, N, D))
    for i in range(1, B1):
        H[i] = H[parent[i]] + 0.01 * rng.standard_normal((N, D))
        H[i, i % N] += 5.0        # one recomputed slot per draft
    rec, src, *_ = F.fold_gate(H, parent, 0.1)
    o, _ = F.attention_folded(q, kb, vb, kc, vc, src, 0.35)
    qr = F.resolve_tables(q, kb, vb, src)[0]
    o_bad, _ = O.attention(qr, kb, vb, kc, vc, 0.35)
    assert np.max(np.abs(o_bad - o)) > 1e-3


def test_synthetic_layer_input_structure():
    """The synthetic layer-input hidden states put committed slots well below
    delta = 0.1, newly unmasked slots near rho = 1, masked slots on both sides."""
    wl = synth.WORKLOADS[2]
    x = synth.draw_inputs(wl, with_w=False)
    H = synth.draw_fold_hidden(wl, x["parent"], x["state"])
    assert H.shape == (wl.B1, wl.N, wl.D)
    num, den = F.fold_residual(synth.bf16_bits_to_f32(H), x["parent"])
    rho = np.sqrt(num[1:] / den[1:])
    st, par = x["state"], x["parent"]
    committed = st[par[1:]] != O.MASK
    fresh = (st[par[1:]] == O.MASK) & (st[1:] != O.MASK)
    masked = st[1:] == O.MASK
    assert np.all(rho[committed] < 0.06)
    assert np.all(rho[fresh] > 0.9)
    assert 0.2 < np.mean(rho[masked] <= 0.1) < 0.8
    rec, *_ = F.fold_gate(synth.bf16_bits_to_f32(H), par, 0.1)
    assert 0.4 < F.fold_ratio(rec) < 0.95
