"""Pins of the oracle LM head (O5): brute-force loops on tiny inputs, one-hot
rows select a weight column exactly, torch CPU matmul as a library routine,
masked-row order (O4)."""
import numpy as np
import torch

from oracle import oracle as O


def test_masked_rows_lexicographic():
    st = np.array([[-1, 3, -1], [4, -1, 5], [1, 2, 3]])
    assert list(O.masked_rows(st)) == [0, 2, 4]
    assert O.masked_rows(np.array([[1, 2]])).size == 0


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    hidden = rng.standard_normal((6, 5))
    w = rng.standard_normal((7, 5))
    rows = np.array([1, 4, 5])
    got = O.lm_head(hidden, rows, w, v_chunk=3)
    for r, row in enumerate(rows):
        for v in range(7):
            acc = 0.0
            for k in range(5):
                acc += hidden[row, k] * w[v, k]
            assert abs(got[r, v] - acc) < 1e-12


def test_one_hot_row_selects_column():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((50, 16))
    hidden = np.zeros((3, 16)); hidden[1, 9] = 1.0
    got = O.lm_head(hidden, np.array([1]), w, v_chunk=13)
    assert np.array_equal(got[0], w[:, 9])


def test_against_torch_matmul():
    rng = np.random.default_rng(2)
    hidden = rng.standard_normal((40, 64))
    w = rng.standard_normal((300, 64))
    rows = np.array([0, 3, 17, 39])
    ref = (torch.from_numpy(hidden[rows]) @ torch.from_numpy(w).T).numpy()
    np.testing.assert_allclose(O.lm_head(hidden, rows, w, v_chunk=128), ref, atol=1e-12)
