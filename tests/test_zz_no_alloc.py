"""sfv_commit_noalloc, the commit with the library's static device workspace,
against sfv_commit with a caller workspace, through the C ABI: tokens,
committed positions, next states and confidences bit-identical, on calls in
a row whose shapes shrink (the static array keeps the previous call's
contents, which the next call must not read)."""
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import sfv, synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(seed, B1, N, V, frac):
    rng = np.random.default_rng(seed)
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, B1)]
    state = rng.integers(0, V, (B1, N)).astype(np.int32)
    state[rng.random((B1, N)) < frac] = sfv.SFV_MASK
    rows = np.flatnonzero(state.reshape(-1) == sfv.SFV_MASK).astype(np.int32)
    logits = synth.draw_logits(rows.size, V, seed)
    return parent, state, rows, logits


def _outputs(B1, N, M, k_max):
    return (torch.full((B1, N), -9, dtype=torch.int32, device="cuda"),
            torch.full((B1, k_max), -9, dtype=torch.int32, device="cuda"),
            torch.full((max(M, 1),), -9, dtype=torch.int32, device="cuda"),
            torch.full((max(M, 1),), float("nan"), dtype=torch.float32, device="cuda"))


def _host(outs, M):
    nxt, cpos, tok, conf = outs
    return dict(next_state=nxt.cpu().numpy(), commit_pos=cpos.cpu().numpy(), token=tok[:M].cpu().numpy(),
                conf=conf[:M].cpu().numpy())


@pytest.mark.parametrize("seed", [0, 1])
def test_noalloc_matches_commit(gpu_lib, seed):
    # large to small, both temperatures, a threshold commit last
    cases = [(21, 32, 151936, 0.6, 1.0, 1, 0.0), (5, 16, 4096, 0.5, 0.0, 1, 0.0),
             (9, 32, 2048, 0.7, 0.7, 2, 0.3)]
    prev_need = None
    for k, (B1, N, V, frac, T, k_max, tau) in enumerate(cases):
        parent, state, rows, logits = _inputs(100 * seed + k, B1, N, V, frac)
        M = rows.size
        need = sfv.sfv_commit_workspace_bytes(B1, N, M, V)
        say(f"noalloc case {k}: B1={B1} N={N} V={V} M={M} T={T} k_max={k_max} workspace<={need}")
        if prev_need is not None and k == 1:
            assert need < prev_need      # the second call is the smaller one
        prev_need = need
        st, rw, lg = (torch.from_numpy(a).cuda() for a in (state, rows, logits))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = _outputs(B1, N, M, k_max)
        sfv.sfv_commit(lg, rw, M, st, parent, B1, N, V, T, 7 + seed, 40 + k, 512, k_max, tau, *ref, ws, need)
        got = _outputs(B1, N, M, k_max)
        sfv.sfv_commit_noalloc(lg, rw, M, st, parent, B1, N, V, T, 7 + seed, 40 + k, 512, k_max, tau, *got)
        torch.cuda.synchronize()
        a, b = _host(ref, M), _host(got, M)
        for key in a:
            assert np.array_equal(a[key], b[key]), (k, key)
        assert np.all(b["token"] >= 0) and np.all(np.isfinite(b["conf"]))
