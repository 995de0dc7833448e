"""Greedy commit from the LM head's tile partials (sfv_lm_head_greedy +
sfv_commit_greedy) against the logits sweep (sfv_lm_head + sfv_commit at
T = 0), through the C ABI.

The sweep path is pinned to the oracle bit for bit on seeded host logits
(test_gpu_parity); here the partials path must give the same logits (the same
kernel arithmetic), the same tokens, committed positions and next states, and
confidences within the fast path's bound, on shapes the large-tile kernel
serves from 33 rows on (256-id tiles, one or both row-tile heights), ragged
vocabularies whose last tile is partly past V, at the full SDAR-8B-like and
D3D packed-tray shapes, with the threshold commit, and on planted exact and
near ties that force the fp64 re-decision.  On every case the pair's outputs
are also held to the oracle (oracle.commit on the pair's own fp32 logits,
copied to the host): tokens, committed positions and next states bit-exact,
confidences within 1e-5 relative; and properties of the outputs on their own
logits are checked: each token is the row's first argmax, conf * sum
exp(l - max) = 1 within 1e-5, and each branch commits a position of maximal
confidence."""
import functools
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import sfv, synth
from branch_verify_amd.step import step_for, to_device
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _state(rng, B1, N, M):
    """Block states with exactly M masked positions (every branch keeps at
    least one unmasked position when M < B1 * N)."""
    flat = np.full(B1 * N, 7, dtype=np.int32)
    flat[rng.choice(B1 * N, M, replace=False)] = sfv.SFV_MASK
    return flat.reshape(B1, N)


def _tree(rng, B1):
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, B1)]
    return par


def _run_both(hd, wd, state_d, parent, B1, N, M, D, V, k_max=1, tau=0.0):
    """Both paths on the same device inputs; returns two dicts of host arrays."""
    R = B1 * N
    rows = torch.empty(R, dtype=torch.int32, device="cuda")
    count = torch.empty(1, dtype=torch.int32, device="cuda")
    sfv.sfv_masked_rows(state_d, B1, N, rows, count)
    out = []
    for fused in (False, True):
        logits = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
        nxt = torch.full((B1, N), -9, dtype=torch.int32, device="cuda")
        cpos = torch.full((B1, k_max), -9, dtype=torch.int32, device="cuda")
        tok = torch.full((M,), -9, dtype=torch.int32, device="cuda")
        conf = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            pb = sfv.sfv_lm_head_greedy_bytes(M, V, D)
            assert pb > 0
            parts = torch.empty(pb, dtype=torch.uint8, device="cuda")
            wsb = sfv.sfv_commit_greedy_workspace_bytes(B1, N, M, V)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            sfv.sfv_lm_head_greedy(hd, rows, M, R, wd, D, V, logits, parts, pb)
            sfv.sfv_commit_greedy(parts, pb, D, logits, rows, M, state_d, parent, B1, N, V, k_max, tau,
                                  nxt, cpos, tok, conf, ws, wsb)
        else:
            wsb = sfv.sfv_commit_workspace_bytes(B1, N, M, V)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            sfv.sfv_lm_head(hd, rows, M, R, wd, D, V, logits)
            sfv.sfv_commit(logits, rows, M, state_d, parent, B1, N, V, 0.0, 0, 0, 0, k_max, tau, nxt, cpos,
                           tok, conf, ws, wsb)
        torch.cuda.synchronize()
        out.append(dict(logits=logits, next_state=nxt.cpu().numpy(), commit_pos=cpos.cpu().numpy(),
                        token=tok.cpu().numpy(), conf=conf.cpu().numpy(), rows=rows[:M].cpu().numpy()))
    return out


def _against_oracle(res, state, parent, k_max, tau):
    """The pair's outputs against oracle.commit on the pair's own fp32 logits
    (T = 0): tokens, committed positions and next states bit-exact."""
    lg_host = res["logits"].cpu().numpy()
    rows = O.masked_rows(state)
    assert np.array_equal(res["rows"], rows)
    nxt, cpos, tok, conf, _ = O.commit(lg_host, rows, state, np.asarray(parent), 0.0, 0, 0, 0,
                                       k_max=k_max, tau=tau)
    assert np.array_equal(res["token"], tok), np.flatnonzero(res["token"] != tok)[:10]
    assert np.array_equal(res["commit_pos"], cpos), np.flatnonzero(np.any(res["commit_pos"] != cpos, 1))[:10]
    assert np.array_equal(res["next_state"], nxt)
    if conf.size:
        rel = np.max(np.abs(res["conf"].astype(np.float64) / conf.astype(np.float64) - 1.0))
        assert rel <= 1e-5, rel
    say("greedy pair equals the oracle commit on its own logits")


def _compare(sweep, parts, state, N, k_max, parent=None, tau=0.0):
    if parent is not None:
        _against_oracle(parts, state, parent, k_max, tau)
    assert torch.equal(sweep["logits"], parts["logits"]), "the same kernel arithmetic must give the same logits"
    assert np.array_equal(sweep["token"], parts["token"])
    assert np.array_equal(sweep["commit_pos"], parts["commit_pos"])
    assert np.array_equal(sweep["next_state"], parts["next_state"])
    rel = np.abs(parts["conf"].astype(np.float64) / sweep["conf"].astype(np.float64) - 1.0)
    assert rel.max() <= 2e-5
    # properties on the logits themselves
    lg = parts["logits"]
    assert np.array_equal(parts["token"], torch.argmax(lg, dim=1).int().cpu().numpy())
    l64 = lg.double()
    S = torch.exp(l64 - l64.max(dim=1, keepdim=True).values).sum(dim=1).cpu().numpy()
    assert np.max(np.abs(parts["conf"] * S - 1.0)) <= 1e-5
    where = {int(r): k for k, r in enumerate(parts["rows"])}
    B1 = state.shape[0]
    for i in range(B1):
        masked = [n for n in range(N) if state[i, n] == sfv.SFV_MASK]
        n0 = int(parts["commit_pos"][i, 0])
        if not masked:
            assert n0 == -1
            continue
        Smin = min(S[where[i * N + n]] for n in masked)
        assert n0 in masked and S[where[i * N + n0]] <= Smin * (1 + 1e-12)
        ties = [n for n in masked if S[where[i * N + n]] == Smin]
        if len(ties) > 1:
            assert n0 == min(ties)


@pytest.mark.parametrize("B1,N,M,D,V,k_max,tau", [
    (5, 32, 129, 128, 1000, 1, 0.0),
    (6, 32, 150, 192, 4104, 1, 0.0),
    (8, 32, 200, 256, 2056, 3, 0.5),
    (8, 32, 256, 128, 1024, 1, 0.0),
    (9, 32, 160, 320, 6216, 2, 0.0),
    (3, 64, 190, 128, 136, 4, 0.9),
    (2, 32, 33, 128, 1000, 1, 0.0),
    (4, 32, 64, 4096, 2056, 1, 0.0),
    (5, 32, 100, 192, 777 // 8 * 8, 2, 0.5),
    (7, 32, 170, 192, 1000, 1, 0.0),
    (7, 32, 224, 4096, 2056, 2, 0.5),
    (9, 32, 257, 64, 1000, 1, 0.0),
    (12, 32, 384, 4096, 4104, 1, 0.0),
    (14, 32, 402, 192, 2056, 2, 0.5),
    (24, 32, 700, 128, 520, 3, 0.9),
    (12, 32, 384, 256, 33288, 1, 0.0),
    (20, 32, 600, 320, 40000, 2, 0.5),
    # more than 256 vocab tiles for one row tile
    (5, 32, 150, 128, 70000, 1, 0.0),
    (9, 32, 148, 64, 151936, 2, 0.5),
])
def test_partials_match_sweep(gpu_lib, B1, N, M, D, V, k_max, tau):
    rng = np.random.default_rng(M * 7 + V)
    say(f"greedy partials B1={B1} N={N} M={M} D={D} V={V} k_max={k_max} tau={tau}")
    R = B1 * N
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((R, D), dtype=np.float32))
    scale = np.exp(rng.uniform(np.log(0.02), np.log(0.3), (V, 1))).astype(np.float32)
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, D)).astype(np.float32) * scale))
    state = _state(rng, B1, N, M)
    parent = _tree(rng, B1)
    hd = torch.from_numpy(hidden).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).view(torch.bfloat16).cuda()
    sd = torch.from_numpy(state).cuda()
    a, b = _run_both(hd, wd, sd, parent, B1, N, M, D, V, k_max, tau)
    _compare(a, b, state, N, k_max, parent, tau)
    a2, b2 = _run_both(hd, wd, sd, parent, B1, N, M, D, V, k_max, tau)
    for k in ("token", "commit_pos", "next_state", "conf"):
        assert np.array_equal(b[k], b2[k]), f"{k} differs between two identical runs"


def test_planted_ties_take_the_lowest_position(gpu_lib):
    """Branch i's masked positions a_i < b_i get the same hidden row, scaled up
    so that they are the branch's most confident: equal logits, equal S, and
    the fp64 re-decision must commit a_i.  A second pair differs by one bf16
    ulp in one element (a near tie the fast bound cannot separate)."""
    rng = np.random.default_rng(5)
    B1, N, D, V = 8, 32, 128, 2048
    M = 170
    R = B1 * N
    state = _state(rng, B1, N, M)
    hid = rng.standard_normal((R, D), dtype=np.float32)
    pairs = []
    for i in range(B1):
        masked = [n for n in range(N) if state[i, n] == sfv.SFV_MASK]
        if len(masked) < 2:
            continue
        a_, b_ = sorted(rng.choice(masked, 2, replace=False))
        base = rng.standard_normal(D).astype(np.float32) * 4.0
        hid[i * N + a_] = base
        hid[i * N + b_] = base
        if i % 2 == 1:  # near tie: one element one bf16 step apart
            bits = synth.f32_to_bf16_bits(base[None])[0].copy()
            bits[3] = bits[3] + 1
            hid[i * N + b_] = synth.bf16_bits_to_f32(bits[None])[0]
        pairs.append((i, int(a_), int(b_), i % 2 == 0))
    hidden = synth.f32_to_bf16_bits(hid)
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, D)) * 0.05).astype(np.float32))
    parent = _tree(rng, B1)
    hd = torch.from_numpy(hidden).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).view(torch.bfloat16).cuda()
    sd = torch.from_numpy(state).cuda()
    say(f"planted ties: {len(pairs)} branches")
    a, b = _run_both(hd, wd, sd, parent, B1, N, M, D, V)
    _compare(a, b, state, N, 1, parent)
    for i, a_, b_, exact in pairs:
        if exact:
            assert b["commit_pos"][i, 0] == a_, (i, a_, b_, b["commit_pos"][i, 0])


@functools.lru_cache(maxsize=1)
def _workload2():
    return synth.draw_inputs(synth.WORKLOADS[2])


def test_partials_match_sweep_full_shape(gpu_lib):
    """The SDAR-8B-like budget-8 workload (M = 148, D = 4096, V = 151936): the
    benchmark's step, greedy, through both paths."""
    wl = synth.WORKLOADS[2]
    x = _workload2()
    xd = to_device(x)
    M = int((x["state"] == sfv.SFV_MASK).sum())
    say(f"greedy partials at the full shape M={M}")
    a, b = _run_both(xd["hidden"], xd["w"], xd["state"], [int(p) for p in x["parent"]], wl.B1, wl.N, M, wl.D,
                     wl.V)
    _compare(a, b, x["state"], wl.N, 1, x["parent"])
    step = step_for(wl, x)
    assert step.fuse, "the benchmark's greedy step runs on the tile partials"
    del xd, step
    torch.cuda.empty_cache()


def test_partials_match_sweep_packed_trays_shape(gpu_lib):
    """The D3D-style packed workload (24 trays x 16, all masked: M = 384, D = 4096,
    V = 151936), greedy: the large-tile LM head with two 192-row tiles writes the
    partials, and both paths must agree."""
    wl = synth.WORKLOADS[4]
    x = synth.draw_inputs(wl)
    xd = to_device(x)
    M = int((x["state"] == sfv.SFV_MASK).sum())
    assert M == 384
    say(f"greedy partials at the packed-tray shape M={M}")
    a, b = _run_both(xd["hidden"], xd["w"], xd["state"], [int(p) for p in x["parent"]], wl.B1, wl.N, M, wl.D,
                     wl.V)
    _compare(a, b, x["state"], wl.N, 1, x["parent"])
    step = step_for(wl, x)
    assert step.fuse, "the packed-tray greedy step runs on the tile partials"
    del xd, step
    torch.cuda.empty_cache()
