"""Every one of the 2^32 noise words: the Gumbel value the device's exact
path decides with (sfv_gumbel_words, fl32(-ln(-ln u)) with fp64 logarithms)
is bit-identical to the oracle's gumbel_from_words (numpy's fp64 log).

The commit's Gumbel-max keys and the drafter's tokens at T > 0 are
fl32(fl32(l * invT) + g); a single word whose fp32 g rounded differently on
the two sides could change a token, so the two implementations are compared
exhaustively rather than on the ids a test happens to draw (SPOT, "Is the
output exact when the target samples?", Proposition 2: drafter and target
must draw the same noise)."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import oracle as O

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27      # words per device call
SUB = 1 << 23        # words per host worker task


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _oracle_bits(first, n):
    w = (np.arange(n, dtype=np.uint64) + np.uint64(first)).astype(np.uint32)
    return O.gumbel_from_words(w).view(np.uint32)


def test_gumbel_exact_matches_oracle_on_every_word(gpu_lib):
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    total = 1 << 32
    bad_words = []
    n_bad = 0
    with ThreadPoolExecutor(max_workers=8) as ex:
        for first in range(0, total, CHUNK):
            gpu_lib.sfv_gumbel_words(first, CHUNK, out)
            dev = out.cpu().numpy().view(np.uint32)
            ref = np.concatenate([f.result() for f in
                                  [ex.submit(_oracle_bits, first + s, SUB) for s in range(0, CHUNK, SUB)]])
            diff = np.flatnonzero(dev != ref)
            n_bad += diff.size
            bad_words += [int(first + d) for d in diff[:8]]
            if (first // CHUNK) % 8 == 7:
                say(f"noise words up to {first + CHUNK:#x}: {n_bad} mismatches so far")
    say(f"all 2^32 words compared: {n_bad} mismatches; first ones {bad_words[:8]}")
    assert n_bad == 0, bad_words[:16]


def test_gumbel_words_edges(gpu_lib):
    """The range ends: the smallest and largest words (u nearest 0 and 1), a
    short ragged call, and an empty one."""
    out = torch.full((5,), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.sfv_gumbel_words(0, 2, out)
    gpu_lib.sfv_gumbel_words(2**32 - 3, 3, out[2:])
    gpu_lib.sfv_gumbel_words(7, 0, out)
    got = out.cpu().numpy()
    want = O.gumbel_from_words(np.array([0, 1, 2**32 - 3, 2**32 - 2, 2**32 - 1], dtype=np.uint32))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert got[0] < got[1] < got[2] < got[3] < got[4]
