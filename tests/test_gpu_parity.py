"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Acceptance (same seeded inputs on both sides):
  * commit and match: tokens, committed positions, next states and matched
    draft indices bit-exact given the same fp32 logits: the step's own LM-head
    logits (copied to the host, fed to the oracle; at T = 0 with 33 or more
    masked rows these come from the fused LM head + greedy commit pair that
    the benchmark times), and seeded fp32 logits drawn on the host;
  * attention: O within 2e-2 max-abs (bf16 in, fp32 accumulation), LSE within
    1e-5 relative;
  * LM-head logits within 3e-2 max-abs.
Sizes the oracle finishes in seconds are compared element by element; the
full workloads are compared on sampled outputs the oracle computes one by one,
in the launch configuration the benchmark times.  Every GPU call is run twice
and must be bit-identical (no atomics feed any decision)."""
import functools
import math
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import synth
from branch_verify_amd.step import VerifyStep, step_for, to_device
from oracle import oracle as O

pytestmark = pytest.mark.gpu

ATT_ABS = 2e-2
LSE_REL = 1e-5
LOGIT_ABS = 3e-2
f32 = synth.bf16_bits_to_f32


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=1)
def host_inputs(idx):
    return synth.draw_inputs(synth.WORKLOADS[idx])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def oracle_attention_rows(x, samples, scale):
    """Oracle O and LSE for sampled (i, n, h), one row at a time."""
    q, kb, vb, kc, vc = (f32(x[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx"))
    G = q.shape[2] // kb.shape[2]
    outs, lses = [], []
    for (i, n, h) in samples:
        g = h // G
        o, l = O.attention(q[i:i + 1, n:n + 1, h:h + 1], kb[i:i + 1, :, g:g + 1],
                           vb[i:i + 1, :, g:g + 1], kc[g:g + 1], vc[g:g + 1], scale)
        outs.append(o[0, 0, 0])
        lses.append(l[0, 0, 0])
    return np.array(outs), np.array(lses)


def check_attention(x, step, full):
    o_gpu = step.o.float().cpu().numpy()
    lse_gpu = step.lse.cpu().numpy()
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    if full:
        o_ref, lse_ref = O.attention(*(f32(x[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")),
                                     step.scale)
        err_o = np.max(np.abs(o_gpu - o_ref))
        err_l = np.max(np.abs(lse_gpu - lse_ref) / np.abs(lse_ref))
    else:
        rng = np.random.default_rng(0)
        B1, N, Hq = lse_gpu.shape
        samples = [(int(rng.integers(B1)), int(rng.integers(N)), int(rng.integers(Hq))) for _ in range(192)]
        samples += [(0, 0, 0), (B1 - 1, N - 1, Hq - 1), (B1 - 1, 0, Hq // 2)]
        o_ref, lse_ref = oracle_attention_rows(x, samples, step.scale)
        og = np.array([o_gpu[s] for s in samples])
        lg = np.array([lse_gpu[s] for s in samples])
        err_o = np.max(np.abs(og - o_ref))
        err_l = np.max(np.abs(lg - lse_ref) / np.abs(lse_ref))
    say(f"attention max|dO|={err_o:.3e} max rel dLSE={err_l:.3e}")
    assert err_o <= ATT_ABS
    assert err_l <= LSE_REL


# ---------------------------------------------------------------------------
# LM head
# ---------------------------------------------------------------------------
def check_lm_head(x, res, full):
    rows = O.masked_rows(x["state"])
    assert np.array_equal(res["rows"], rows)
    logits = res["logits"]
    M, V = logits.shape
    hidden = f32(x["hidden"])
    if full:
        ref = O.lm_head(hidden, rows, f32(x["w"]))
        got = logits.cpu().numpy()
        err = np.max(np.abs(got - ref))
    else:
        rng = np.random.default_rng(1)
        rsel = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 14)]))
        cols = np.unique(np.concatenate([np.arange(256), np.arange(V - 256, V),
                                         rng.integers(0, V, 4096),
                                         np.arange(127, V, 128)[:64], np.arange(128, V, 128)[-64:]]))
        w = f32(x["w"][cols])
        ref = hidden[rows[rsel]].astype(np.float64) @ w.astype(np.float64).T
        got = logits[torch.from_numpy(rsel).to(logits.device)][:, torch.from_numpy(cols).to(logits.device)]
        err = np.max(np.abs(got.cpu().numpy() - ref))
    say(f"lm_head max|dlogit|={err:.3e}")
    assert err <= LOGIT_ABS


# ---------------------------------------------------------------------------
# commit and match
# ---------------------------------------------------------------------------
def check_commit_match(x, res, wl_T, seed, step0, pos0, S_max, logits_host, k_max=1, tau=0.0):
    rows = O.masked_rows(x["state"])
    assert np.array_equal(res["rows"], rows)
    lg = logits_host
    nxt, cpos, tok, conf, S = O.commit(lg, rows, x["state"], x["parent"], wl_T, seed, step0, pos0,
                                       k_max=k_max, tau=tau)
    assert np.array_equal(res["token"], tok), np.flatnonzero(res["token"] != tok)[:10]
    assert res["commit_pos"].shape == cpos.shape
    assert np.array_equal(res["commit_pos"], cpos), np.flatnonzero(np.any(res["commit_pos"] != cpos, 1))[:10]
    assert np.array_equal(res["next_state"], nxt)
    rel = np.max(np.abs(res["conf"].astype(np.float64) - conf.astype(np.float64)) / conf) if conf.size else 0.0
    say(f"commit tokens/positions exact; conf max rel err {rel:.2e}")
    assert rel <= 1e-5
    chain, h, status = O.match_tree(x["state"], nxt, cpos, x["parent"], S_max)
    assert res["status"] == status
    assert res["h"] == h
    assert np.array_equal(res["chain"], chain)
    return h


def commit_on(step, xd, lg_host):
    """Commit and walk of `step` on host logits; returns results like step.results()."""
    lg = torch.from_numpy(lg_host).cuda()
    step.commit(xd, logits=lg)
    step.match(xd)
    torch.cuda.synchronize()
    res = step.results()
    del lg
    return res


def run_twice(step, xd):
    """The step overlapped (attention on a second stream, beside the commit),
    then in order on one stream: every output must be bit-identical."""
    step.run(xd, attn_with="commit")
    first = step.results()
    snap = {k: (v.clone() if torch.is_tensor(v) else np.copy(v) if isinstance(v, np.ndarray) else v)
            for k, v in first.items()}
    step.run(xd, overlap=False)
    second = step.results()
    for k in snap:
        a, b = snap[k], second[k]
        if torch.is_tensor(a):
            assert torch.equal(a, b), f"{k} differs between two identical runs"
        elif isinstance(a, np.ndarray):
            assert np.array_equal(a, b), f"{k} differs between two identical runs"
        else:
            assert a == b, k
    return second


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_full_step_parity(gpu_lib, idx):
    wl = synth.WORKLOADS[idx]
    say(f"workload {idx} {wl.name}: drawing inputs")
    x = host_inputs(idx)
    xd = to_device(x)
    step = step_for(wl, x)
    say(f"workload {idx}: B1={wl.B1} N={wl.N} L={wl.L} M={step.M} running the step twice")
    res = run_twice(step, xd)
    assert res["count"] == step.M
    assert np.array_equal(res["rows"], O.masked_rows(x["state"]))
    check_attention(x, step, full=idx <= 4)
    check_lm_head(x, res, full=idx == 1)
    # the step's commit and walk on its own logits (the greedy pair at c2 and
    # c4), against the oracle on those logits
    say(f"workload {idx}: oracle commit + match on the step's own logits (fused={step.fuse})")
    check_commit_match(x, res, wl.T, wl.seed, wl.step0, wl.pos0, wl.S_t,
                       logits_host=res["logits"].cpu().numpy())
    # the commit and the walk at this shape on seeded host logits, against the oracle
    lg = synth.draw_logits(step.M, wl.V, wl.seed)
    say(f"workload {idx}: commit + match on seeded logits")
    res2 = commit_on(step, xd, lg)
    check_commit_match(x, res2, wl.T, wl.seed, wl.step0, wl.pos0, wl.S_t, logits_host=lg)
    del xd, step
    torch.cuda.empty_cache()


@pytest.mark.parametrize("attn_with", ["auto", "lm_head", "commit"])
@pytest.mark.parametrize("idx", [2, 3])
def test_graph_replay_matches_eager(gpu_lib, idx, attn_with):
    """The whole step captured in a HIP graph, with the attention in order or
    on a second stream beside the LM head or the commit: every replay (with
    eager work and synchronisation between replays, and the outputs
    overwritten before each) reproduces the eager in-order step bit for bit."""
    wl = synth.WORKLOADS[idx]
    say(f"graph replay, workload {idx}, attention {attn_with}")
    x = host_inputs(idx)
    xd = to_device(x)
    step = step_for(wl, x)
    step.run(xd, overlap=False)
    ref = {k: (v.clone() if torch.is_tensor(v) else np.copy(v) if isinstance(v, np.ndarray) else v)
           for k, v in step.results().items()}
    step.capture(xd, attn_with=attn_with)
    outs = [step.o, step.lse, step.logits, step.next_state, step.commit_pos, step.token, step.conf,
            step.chain, step.n_accepted, step.status, step.rows, step.count]
    for rep in range(3):
        for t in outs:  # eager work between replays: poison every output
            t.fill_(-7 if not t.is_floating_point() else float("nan"))
        torch.cuda.synchronize()
        step.replay()
        got = step.results()
        for k, a in ref.items():
            b = got[k]
            if torch.is_tensor(a):
                assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager step"
            elif isinstance(a, np.ndarray):
                assert np.array_equal(a, b), f"replay {rep}: {k} differs from the eager step"
            else:
                assert a == b, (rep, k)
    del xd, step
    torch.cuda.empty_cache()


def test_selfcheck_bounds(gpu_lib):
    out = torch.zeros(2, dtype=torch.float64, device="cuda")
    say("self-check: all 2^32 noise words and all fp32 exp2 arguments in [-126, 6]")
    gpu_lib.sfv_selfcheck_bounds(out)
    torch.cuda.synchronize()
    g_err, e_rel = out.cpu().tolist()
    say(f"max excess of g over its bucket's bounds = {g_err:.3e}; max rel err exp2 = {e_rel:.3e}")
    assert g_err == 0.0                      # every word's exact noise inside its bucket
    assert e_rel < 2.0 ** -22                # commit error model uses 2^-20


# ---------------------------------------------------------------------------
# commit + match on planted trees (toy target; SPOT Propositions 1-2)
# ---------------------------------------------------------------------------
def _planted_case(rng, N, V, T, step0, pos0, seed, depth, decoys, k_max=1, tau=0.0):
    s0 = rng.integers(0, V, N).astype(np.int32)
    s0[rng.choice(N, max(depth + 2, N // 2), replace=False)] = O.MASK
    traj = [s0]
    for t in range(depth):
        cur = traj[-1][None]
        rows = O.masked_rows(cur)
        lg = synth.state_keyed_logits(seed, cur[0], V)[rows]
        nxt, *_ = O.commit(lg, rows, cur, np.array([-1]), T, seed, step0 + t, pos0, k_max=k_max, tau=tau)
        traj.append(nxt[0])
    states, parent = [traj[0]], [-1]
    for t in range(1, len(traj)):
        parent.append(len(states) - 1)
        states.append(traj[t])
    for _ in range(decoys):
        p = int(rng.integers(0, len(states)))
        row = states[p].copy()
        free = np.flatnonzero(row == O.MASK)
        if free.size == 0:
            continue
        row[int(rng.choice(free))] = int(rng.integers(0, V))
        if any(np.array_equal(row, s) for s in traj):
            continue
        states.append(row)
        parent.append(p)
    st = np.stack(states).astype(np.int32)
    return st, np.array(parent, dtype=np.int32), len(traj) - 1


def _run_commit_match(st, parent, V, T, seed, step0, pos0, logits_host, S_max=1, k_max=1, tau=0.0):
    B1, N = st.shape
    rows = O.masked_rows(st)
    M = rows.size
    step = VerifyStep(B1, N, 0, 1, 1, 32, 64, V, M, parent, T, seed, step0, pos0, S_max=S_max,
                      k_max=k_max, tau=tau)
    xd = {"state": torch.from_numpy(st).cuda()}
    step.masked_rows(xd)
    lg = torch.from_numpy(np.ascontiguousarray(logits_host)).cuda()
    step.commit(xd, logits=lg)
    step.match(xd)
    torch.cuda.synchronize()
    res = dict(rows=step.rows[:M].cpu().numpy(), logits=lg, token=step.token[:M].cpu().numpy(),
               conf=step.conf[:M].cpu().numpy(), commit_pos=step.commit_pos.cpu().numpy(),
               next_state=step.next_state.cpu().numpy(), chain=step.chain.cpu().numpy(),
               h=int(step.n_accepted.item()), status=int(step.status.item()))
    return res


@pytest.mark.parametrize("T", [0.0, 1.0, 0.7])
@pytest.mark.parametrize("case", range(4))
def test_planted_chain_match(gpu_lib, T, case):
    rng = np.random.default_rng(300 + case)
    N, V, seed = [8, 32, 16, 64][case], [512, 151936, 4096, 2048][case], 77 + case
    step0, pos0 = 900 + case, 4096
    depth = int(rng.integers(1, 6))
    st, parent, planted = _planted_case(rng, N, V, T, step0, pos0, seed, depth, decoys=int(rng.integers(3, 20)))
    say(f"planted case {case} T={T} B1={st.shape[0]} N={N} V={V} depth={depth}")
    rows = O.masked_rows(st)
    lg = np.stack([synth.state_keyed_logits(seed, st[r // N], V)[r % N] for r in rows])
    res = _run_commit_match(st, parent, V, T, seed, step0, pos0, lg)
    x = dict(state=st, parent=parent)
    h = check_commit_match(x, res, T, seed, step0, pos0, 1, logits_host=lg)
    assert h == planted


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("case", range(3))
def test_mixed_depth_tree_match(gpu_lib, T, case):
    """Drafts holding draft-free states at other tree depths than their step
    count (copies of their parent, or two steps ahead of it): the walk takes
    only drafts one level below the current branch, as the oracle does, and
    the final state equals draft-free decoding for h + 1 steps."""
    rng = np.random.default_rng(520 + case)
    N, V, seed = [8, 32, 64][case], [512, 4096, 151936][case], 91 + case
    step0, pos0 = 70 + case, 2048
    s0 = rng.integers(0, V, N).astype(np.int32)
    s0[rng.choice(N, 7, replace=False)] = O.MASK

    def decode_free(steps):
        traj = [s0]
        for t in range(steps):
            cur = traj[-1][None]
            rows = O.masked_rows(cur)
            if rows.size == 0:
                break
            lg1 = synth.state_keyed_logits(seed, cur[0], V)[rows]
            nxt1, *_ = O.commit(lg1, rows, cur, np.array([-1]), T, seed, step0 + t, pos0)
            traj.append(nxt1[0])
        return traj

    traj = decode_free(7)
    st, par, t_of = [traj[0]], [-1], [0]
    B1 = int(rng.integers(12, 40))
    while len(st) < B1:
        p = int(rng.integers(0, len(st)))
        if t_of[p] < 0 or rng.random() < 0.2:
            row = st[p].copy()
            free = np.flatnonzero(row == O.MASK)
            if free.size == 0:
                continue
            row[int(rng.choice(free))] = int(rng.integers(0, V))
            if any(np.array_equal(row, q) for q in traj):
                continue
            st.append(row); par.append(p); t_of.append(-1)
            continue
        t = min(len(traj) - 1, t_of[p] + int(rng.integers(0, 3)))
        st.append(traj[t].copy()); par.append(p); t_of.append(t)
    st, parent = np.stack(st).astype(np.int32), np.array(par, np.int32)
    say(f"mixed-depth tree case {case} T={T} B1={B1} N={N} V={V}")
    rows = O.masked_rows(st)
    lg = np.stack([synth.state_keyed_logits(seed, st[r // N], V)[r % N] for r in rows])
    res = _run_commit_match(st, parent, V, T, seed, step0, pos0, lg, S_max=2)
    h = check_commit_match(dict(state=st, parent=parent), res, T, seed, step0, pos0, 2, logits_host=lg)
    final = res["next_state"][0 if h == 0 else int(res["chain"][h - 1])]
    assert np.array_equal(final, decode_free(h + 1)[-1])


def test_tie_breaks(gpu_lib):
    V, N = 2048, 6
    rng = np.random.default_rng(5)
    st = np.array([[-1, -1, -1, 4, -1, 9],
                   [7, -1, -1, 4, -1, 9],
                   [7, -1, -1, 4, -1, 9],      # duplicate draft of branch 1
                   [-1, -1, -1, 4, 3, 9]], np.int32)
    parent = np.array([-1, 0, 0, 0], np.int32)
    rows = O.masked_rows(st)
    lg = (rng.standard_normal((rows.size, V)) * 1.28).astype(np.float32)
    r00, r01, r02 = 0, 1, 2
    lg[r01] = lg[r00]                  # identical rows -> equal S -> lower position wins
    lg[r02, 11] = lg[r02].max() + 2.0  # a third, clearly less confident position
    lg[r00, 7] = lg[r00].max() + 6.0   # token 7, very confident
    lg[r01, 7] = lg[r01].max() + 6.0
    lg[r00, 5] = lg[r00, 7]            # token tie at T = 0 -> lowest id (5)
    lg[r01, 5] = lg[r01, 7]
    x = dict(state=st, parent=parent)
    for T in (0.0, 1.0):
        res = _run_commit_match(st, parent, V, T, 3, 40, 100, lg)
        check_commit_match(x, res, T, 3, 40, 100, 1, logits_host=lg)
    res = _run_commit_match(st, parent, V, 0.0, 3, 40, 100, lg)
    assert res["commit_pos"][0, 0] == 0 and res["token"][0] == 5


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_commit_ramped_logits(gpu_lib, T):
    """Logits that rise along the vocabulary by more than 4 per 2048 ids (a
    lane's step), so every lane's running max keeps moving and the sampled
    sweep's confidence sums are rescaled at every iteration; falling and
    sawtooth rows beside them, and in branch 1 two masked positions with
    identical logits (equal confidence: the lower position is committed).  A
    chain of 8 branches of 64 positions, all masked (M = 512), over the full
    vocabulary: the sweep takes 4 vocab ranges of 19 iterations.  Tokens,
    positions and the walk are the oracle's; conf within 1e-5."""
    rng = np.random.default_rng(4321)
    B1, N, V = 8, 64, 151936
    st = np.full((B1, N), O.MASK, np.int32)
    parent = np.arange(-1, B1 - 1, dtype=np.int32)
    rows = O.masked_rows(st)
    ramp = np.arange(V, dtype=np.float32) * np.float32(6.0 / 2048)
    saw = (np.arange(V) % 8192).astype(np.float32) * np.float32(30.0 / 8192)
    shapes = [ramp, ramp[::-1].copy(), saw]
    lg = np.stack([rng.standard_normal(V).astype(np.float32) + shapes[k % 3]
                   for k in range(rows.size)]).astype(np.float32)
    ra, rb = 1 * N + 2, 1 * N + 9  # rows are (i, n) in order: all positions are masked
    lg[rb] = lg[ra]
    lg[ra, 77] = lg[ra].max() + 8.0  # branch 1's most confident positions, tied
    lg[rb, 77] = lg[ra, 77]
    say(f"ramped logits T={T} B1={B1} N={N} M={rows.size} V={V}")
    x = dict(state=st, parent=parent)
    res = _run_commit_match(st, parent, V, T, 11, 500, 64, lg)
    check_commit_match(x, res, T, 11, 500, 64, 1, logits_host=lg)
    assert res["commit_pos"][1, 0] == 2


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_gumbel_key_near_ties(gpu_lib, T):
    """Thousands of ids per row whose Gumbel keys fl32(fl32(l/T) + g) lie
    within a few ulps of each other, many exactly equal: the sweep's screen
    by per-bucket noise bounds must pass every one of them to the exact path,
    and the token is the first argmax (lowest id on ties), as the oracle."""
    V, N = 65536, 8
    seed, step0, pos0 = 11, 70, 300
    st = np.array([[-1, -1, 3, -1, -1, 5, -1, -1],
                   [-1, 8, 3, -1, -1, 5, -1, -1],
                   [-1, -1, 3, 2, -1, 5, -1, -1],
                   [-1, 8, 3, -1, 6, 5, -1, -1]], np.int32)
    parent = np.array([-1, 0, 0, 1], np.int32)
    depth = O.tree_depths(parent)
    rows = O.masked_rows(st)
    rng = np.random.default_rng(17)
    lg = (rng.standard_normal((rows.size, V)) * 1.3).astype(np.float32)
    inv_t = np.float32(1.0) / np.float32(T)
    for r, flat in enumerate(rows):
        i, n = divmod(int(flat), N)
        g = O.gumbel(seed, step0 + int(depth[i]), pos0 + n, np.arange(V)).astype(np.float64)
        planted = rng.choice(V, 3000, replace=False)
        # fl32(l / T) ~ 40 - g: keys within a few ulps of 40
        lg[r, planted] = ((40.0 - g[planted]) * T).astype(np.float32)
        keys = (lg[r] * inv_t).astype(np.float32) + O.gumbel(seed, step0 + int(depth[i]), pos0 + n, np.arange(V))
        top = keys.max()
        say(f"T={T} row {r}: {int(np.sum(keys == top))} ids at the max key, "
            f"{int(np.sum(keys >= top - 4 * np.spacing(np.float32(40))))} within 4 ulps")
    x = dict(state=st, parent=parent)
    res = _run_commit_match(st, parent, V, T, seed, step0, pos0, lg)
    check_commit_match(x, res, T, seed, step0, pos0, 1, logits_host=lg)


def test_duplicate_draft_lowest_index(gpu_lib):
    V, N = 1024, 4
    st0 = np.array([-1, -1, 2, 3], np.int32)
    rows0 = O.masked_rows(st0[None])
    lg0 = synth.state_keyed_logits(11, st0, V)[rows0]
    nxt, *_ = O.commit(lg0, rows0, st0[None], np.array([-1]), 0.0, 11, 5, 0)
    decoy = st0.copy(); decoy[0] = (nxt[0][0] + 1) % V if nxt[0][0] != -1 else 1; decoy[1] = -1
    st = np.stack([st0, decoy, nxt[0], nxt[0], nxt[0]]).astype(np.int32)
    parent = np.array([-1, 0, 0, 0, 0], np.int32)
    rows = O.masked_rows(st)
    lg = np.stack([synth.state_keyed_logits(11, st[r // N], V)[r % N] for r in rows])
    res = _run_commit_match(st, parent, V, 0.0, 11, 5, 0, lg)
    x = dict(state=st, parent=parent)
    check_commit_match(x, res, 0.0, 11, 5, 0, 1, logits_host=lg)
    assert res["chain"][0] == 2


def test_state_violation_status(gpu_lib):
    V, N = 512, 4
    st = np.array([[-1, -1, -1, 3], [1, 2, -1, 3], [1, 5, -1, 3]], np.int32)
    parent = np.array([-1, 0, 0], np.int32)
    rows = O.masked_rows(st)
    lg = np.random.default_rng(1).standard_normal((rows.size, V)).astype(np.float32)
    res = _run_commit_match(st, parent, V, 0.0, 1, 1, 0, lg, S_max=1)
    assert res["status"] == O.SFV_E_STATE and res["h"] == 0 and np.all(res["chain"] == -1)
    res = _run_commit_match(st, parent, V, 0.0, 1, 1, 0, lg, S_max=2)
    assert res["status"] == O.SFV_OK


@pytest.mark.parametrize("hops,dup", [(40, True), (63, False), (0, False)])
def test_match_largest_tree(gpu_lib, hops, dup):
    """sfv_match_tree alone at 64 branches x 256 positions (the largest
    supported tree and block): a planted chain of `hops` drafts, each the
    committed next state of the one before, the others random one-position
    extensions of a random parent; with `dup` one more draft repeats a chain
    state at a higher index, and the lowest must be taken.  hops = 63 walks
    every branch (the B-hop limit); hops = 0 plants nothing."""
    rng = np.random.default_rng(1000 + hops)
    B1, N, V = 64, 256, 1000
    say(f"match largest tree hops={hops} dup={dup}")
    chain = sorted(rng.choice(np.arange(1, B1), hops, replace=False).tolist())
    on_chain = set(chain)
    state = np.empty((B1, N), np.int32)
    nxt = np.empty((B1, N), np.int32)
    cpos = np.empty((B1, 1), np.int32)
    parent = [-1] * B1
    state[0] = rng.integers(0, V, N)
    state[0, rng.random(N) < 0.7] = O.MASK
    prev = 0
    dup_at = None
    for i in range(B1):
        if i > 0:
            if i in on_chain:
                parent[i], state[i] = prev, nxt[prev]
                prev = i
            elif dup and dup_at is None and len([c for c in chain if c < i]) >= 5:
                c5 = [c for c in chain if c < i][4]
                parent[i], state[i] = parent[c5], state[c5]
                dup_at = (i, c5)
            else:
                p = int(rng.integers(0, i))
                parent[i], row = p, state[p].copy()
                free = np.flatnonzero(row == O.MASK)
                row[int(rng.choice(free))] = int(rng.integers(0, V))
                state[i] = row
        free = np.flatnonzero(state[i] == O.MASK)
        n0 = int(rng.choice(free))
        nxt[i] = state[i]
        nxt[i, n0] = int(rng.integers(0, V))
        cpos[i, 0] = n0
    if dup:
        assert dup_at is not None
    st_d, nx_d, cp_d = (torch.from_numpy(a).cuda() for a in (state, nxt, cpos))
    for S_max in (1, -1):
        ch = torch.full((B1,), -9, dtype=torch.int32, device="cuda")
        h = torch.full((1,), -9, dtype=torch.int32, device="cuda")
        status = torch.full((1,), -9, dtype=torch.int32, device="cuda")
        gpu_lib.sfv_match_tree(st_d, nx_d, cp_d, parent, B1, N, 1, S_max, ch, h, status)
        torch.cuda.synchronize()
        ref_chain, ref_h, ref_status = O.match_tree(state, nxt, cpos, np.array(parent), S_max=S_max)
        assert int(status.item()) == ref_status == O.SFV_OK
        assert int(h.item()) == ref_h == hops
        assert np.array_equal(ch.cpu().numpy(), ref_chain)
        assert ref_chain[:hops].tolist() == chain
    # one changed token in a chain state's last position breaks the chain there
    if hops:
        bad = state.copy()
        k = len(chain) // 2
        bad[chain[k], N - 1] = (bad[chain[k], N - 1] + 1) % V if bad[chain[k], N - 1] >= 0 else 3
        ch = torch.full((B1,), -9, dtype=torch.int32, device="cuda")
        h = torch.full((1,), -9, dtype=torch.int32, device="cuda")
        status = torch.full((1,), -9, dtype=torch.int32, device="cuda")
        gpu_lib.sfv_match_tree(torch.from_numpy(bad).cuda(), nx_d, cp_d, parent, B1, N, 1, -1, ch, h, status)
        torch.cuda.synchronize()
        ref_chain, ref_h, _ = O.match_tree(bad, nxt, cpos, np.array(parent), S_max=-1)
        assert int(h.item()) == ref_h
        assert np.array_equal(ch.cpu().numpy(), ref_chain)


# ---------------------------------------------------------------------------
# ragged and degenerate shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [
    dict(B1=5, N=7, L=100, Hq=8, Hkv=1, d=64),
    dict(B1=2, N=1, L=0, Hq=2, Hkv=2, d=32),
    dict(B1=1, N=64, L=1000, Hq=16, Hkv=2, d=128),
    dict(B1=64, N=3, L=70, Hq=4, Hkv=4, d=128),
    dict(B1=3, N=256, L=130, Hq=2, Hkv=1, d=32),
    dict(B1=2, N=5, L=1500, Hq=8, Hkv=2, d=64),   # 2 context splits, the last one ragged
    dict(B1=3, N=9, L=3000, Hq=4, Hkv=4, d=32),   # 5 context splits, the last one ragged
    # unsplit row tiles in whole rounds, then a split tail of the remaining ones
    dict(B1=33, N=64, L=256, Hq=64, Hkv=8, d=128),  # 1024 + 4 x 8 tiles, tail in 2 splits
    dict(B1=61, N=40, L=700, Hq=32, Hkv=4, d=32),   # 600 + 25 x 4 tiles, ragged last tile and split
    dict(B1=4, N=16, L=192, Hq=8, Hkv=2, d=64),     # three full context tiles, no partial one
])
def test_attention_ragged(gpu_lib, shape):
    rng = np.random.default_rng(9)
    B1, N, L, Hq, Hkv, d = (shape[k] for k in ("B1", "N", "L", "Hq", "Hkv", "d"))
    say(f"attention ragged {shape}")
    x = dict(q=synth.f32_to_bf16_bits(rng.standard_normal((B1, N, Hq, d), dtype=np.float32)),
             k_blk=synth.f32_to_bf16_bits(rng.standard_normal((B1, N, Hkv, d), dtype=np.float32)),
             v_blk=synth.f32_to_bf16_bits(rng.standard_normal((B1, N, Hkv, d), dtype=np.float32)),
             k_ctx=synth.f32_to_bf16_bits(rng.standard_normal((Hkv, max(L, 1), d), dtype=np.float32))[:, :L],
             v_ctx=synth.f32_to_bf16_bits(rng.standard_normal((Hkv, max(L, 1), d), dtype=np.float32))[:, :L])
    xd = to_device(x)
    step = VerifyStep(B1, N, L, Hq, Hkv, d, 64, 8, 0, [-1] + [0] * (B1 - 1), 0.0, 1, 1, 0)
    step.attend(xd)
    torch.cuda.synchronize()
    check_attention(x, step, full=True)


@pytest.mark.parametrize("M,D,V", [(1, 64, 8), (5, 128, 1000), (128, 256, 513), (129, 128, 1001),
                                   (130, 192, 1001), (160, 4096, 4100), (193, 320, 2052),
                                   (256, 128, 777), (257, 4096, 2048), (300, 128, 1001),
                                   (513, 192, 777), (300, 64, 1001), (400, 320, 2052),
                                   (1100, 5120, 600), (384, 4096, 2052), (1482, 256, 1000),
                                   (402, 4096, 2052), (700, 192, 1001), (32, 128, 1000),
                                   (33, 128, 1000), (64, 4096, 4100), (100, 192, 777), (128, 64, 999),
                                   (180, 192, 1001), (192, 4096, 3000), (224, 256, 1001), (200, 320, 777),
                                   (300, 256, 33280), (512, 320, 33000), (520, 256, 40001),
                                   (161, 256, 1001), (40, 64, 8), (33, 64, 255), (47, 192, 130),
                                   # more than 256 vocab tiles for one row tile (ragged vocab)
                                   (100, 256, 70001), (192, 128, 65540), (33, 64, 151936)])
def test_lm_head_ragged(gpu_lib, M, D, V):
    rng = np.random.default_rng(M)
    R = M + 3
    say(f"lm_head ragged M={M} D={D} V={V}")
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((R, D), dtype=np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, D)) * 0.05).astype(np.float32))
    rows = np.sort(rng.choice(R, M, replace=False)).astype(np.int32)
    hd = torch.from_numpy(hidden).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).view(torch.bfloat16).cuda()
    rd = torch.from_numpy(rows).cuda()
    out = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.sfv_lm_head(hd, rd, M, R, wd, D, V, out)
    torch.cuda.synchronize()
    ref = O.lm_head(f32(hidden), rows, f32(w))
    err = np.max(np.abs(out.cpu().numpy() - ref))
    assert err <= LOGIT_ABS


@pytest.mark.parametrize("M", [20, 100, 300])
def test_lm_head_row_status(gpu_lib, M):
    """The optional status word of sfv_lm_head / sfv_lm_head_greedy: SFV_OK
    for row ids in [0, R), SFV_E_INVAL when one is outside; the product still
    reads only inside hidden (out-of-range ids read the nearest row) and the
    in-range rows' logits are unchanged."""
    rng = np.random.default_rng(40 + M)
    D, V = 128, 1000
    R = M + 5
    hidden = synth.f32_to_bf16_bits(rng.standard_normal((R, D), dtype=np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((V, D)) * 0.05).astype(np.float32))
    rows = np.sort(rng.choice(R, M, replace=False)).astype(np.int32)
    hd = torch.from_numpy(hidden).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).view(torch.bfloat16).cuda()
    ref = O.lm_head(f32(hidden), rows, f32(w))
    for bad in (None, R, -1, 1 << 30):
        r = rows.copy()
        if bad is not None:
            r[M // 2] = bad
        say(f"lm_head row status M={M} bad id={bad}")
        rd = torch.from_numpy(r).cuda()
        out = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        gpu_lib.sfv_lm_head(hd, rd, M, R, wd, D, V, out, status=st)
        calls = [("lm_head", out, st)]
        if M > 32:
            pb = gpu_lib.sfv_lm_head_greedy_bytes(M, V, D)
            parts = torch.empty(pb, dtype=torch.uint8, device="cuda")
            out2 = torch.full((M, V), float("nan"), dtype=torch.float32, device="cuda")
            st2 = torch.full((1,), 7, dtype=torch.int32, device="cuda")
            gpu_lib.sfv_lm_head_greedy(hd, rd, M, R, wd, D, V, out2, parts, pb, status=st2)
            calls.append(("lm_head_greedy", out2, st2))
        torch.cuda.synchronize()
        for name, o, s_ in calls:
            assert int(s_.item()) == (O.SFV_OK if bad is None else -1), name
            got = o.cpu().numpy()
            assert np.all(np.isfinite(got))
            keep = np.arange(M) != M // 2 if bad is not None else np.ones(M, bool)
            assert np.max(np.abs(got[keep] - ref[keep])) <= LOGIT_ABS, name


@pytest.mark.parametrize("fill", ["none", "all", "random"])
def test_masked_rows_edges(gpu_lib, fill):
    rng = np.random.default_rng(2)
    B1, N = 64, 256
    st = rng.integers(0, 100, (B1, N)).astype(np.int32)
    if fill == "all":
        st[:] = -1
    elif fill == "random":
        st[rng.random((B1, N)) < 0.3] = -1
    rows = torch.full((B1 * N,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.sfv_masked_rows(torch.from_numpy(st).cuda(), B1, N, rows, cnt)
    torch.cuda.synchronize()
    ref = O.masked_rows(st)
    assert int(cnt.item()) == ref.size
    assert np.array_equal(rows[:ref.size].cpu().numpy(), ref)


def test_commit_nothing_masked(gpu_lib):
    st = np.array([[1, 2, 3], [1, 2, 3]], np.int32)
    parent = np.array([-1, 0], np.int32)
    step = VerifyStep(2, 3, 0, 1, 1, 32, 64, 8, 0, parent, 1.0, 1, 1, 0, S_max=0)
    xd = {"state": torch.from_numpy(st).cuda()}
    step.masked_rows(xd)
    step.commit(xd, logits=torch.zeros((1, 8), device="cuda"))
    step.match(xd)
    torch.cuda.synchronize()
    assert np.array_equal(step.next_state.cpu().numpy(), st)
    assert np.all(step.commit_pos.cpu().numpy() == -1)
    assert int(step.n_accepted.item()) == 0


# ---------------------------------------------------------------------------
# threshold commit of up to k_max positions per branch
# ---------------------------------------------------------------------------
def _spread_logits(rng, M, V):
    """Rows of very different sharpness, so confidences spread from about 1/V
    to about 1 and a threshold splits the ranked positions of a branch."""
    scale = np.exp(rng.uniform(np.log(0.3), np.log(12.0), (M, 1)))
    return (rng.standard_normal((M, V)) * scale).astype(np.float32)


@pytest.mark.parametrize("k_max,q", [(2, 0.5), (3, 0.2), (4, 0.8), (8, 0.0), (5, 1.0)])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_threshold_commit_random(gpu_lib, k_max, q, T):
    rng = np.random.default_rng(k_max * 31 + int(10 * q))
    B1, N, V = 9, 32, 4096
    st = rng.integers(0, V, (B1, N)).astype(np.int32)
    st[rng.random((B1, N)) < 0.6] = -1
    st[3] = -1                  # fully masked branch
    st[5, st[5] == -1] = 7      # nothing masked
    parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, B1)], np.int32)
    rows = O.masked_rows(st)
    lg = _spread_logits(rng, rows.size, V)
    *_, conf, _S = O.commit(lg, rows, st, parent, T, 4, 10, 0)
    tau = float(np.quantile(conf, q))
    say(f"threshold commit k_max={k_max} tau={tau:.4g} T={T}")
    res = _run_commit_match(st, parent, V, T, 4, 10, 0, lg, S_max=-1, k_max=k_max, tau=tau)
    check_commit_match(dict(state=st, parent=parent), res, T, 4, 10, 0, -1, logits_host=lg,
                       k_max=k_max, tau=tau)
    taken = np.sum(res["commit_pos"] >= 0, axis=1)
    assert taken[5] == 0 and taken[3] >= 1


def test_threshold_commit_tau_on_boundary(gpu_lib):
    """tau equal to a position's fp32 confidence takes it (>=); one ulp above
    does not: the fast path's bound straddles tau, so S is recomputed exactly."""
    rng = np.random.default_rng(17)
    B1, N, V = 4, 16, 8192
    st = np.full((B1, N), -1, np.int32)
    parent = np.array([-1, 0, 0, 1], np.int32)
    rows = O.masked_rows(st)
    lg = _spread_logits(rng, rows.size, V)
    _n, cpos1, _t, conf, S = O.commit(lg, rows, st, parent, 0.0, 2, 3, 0, k_max=N, tau=-1e30)
    for i in range(B1):
        second = int(cpos1[i, 1])
        c = np.float32(conf[i * N + second])  # rows are the whole block, in order
        for tau, expect_two in ((float(c), True), (float(np.nextafter(c, np.float32(np.inf))), False)):
            res = _run_commit_match(st, parent, V, 0.0, 2, 3, 0, lg, S_max=-1, k_max=2, tau=tau)
            check_commit_match(dict(state=st, parent=parent), res, 0.0, 2, 3, 0, -1, logits_host=lg,
                               k_max=2, tau=tau)
            assert (res["commit_pos"][i, 1] == second) == expect_two


def test_threshold_commit_ties_and_all(gpu_lib):
    """Equal S (identical rows) rank by position; k_max = N with a very low tau
    commits every masked position."""
    rng = np.random.default_rng(23)
    B1, N, V = 3, 12, 2048
    st = np.full((B1, N), -1, np.int32)
    st[1, ::3] = 5
    parent = np.array([-1, 0, 1], np.int32)
    rows = O.masked_rows(st)
    lg = _spread_logits(rng, rows.size, V)
    lg[4, 3] += 30.0                 # a very confident row ...
    lg[[2, 5, 7, 9]] = lg[4]         # ... shared by five positions of branch 0
    for k_max, tau in ((3, 0.0), (5, 0.5), (N, -1e30)):
        say(f"ties k_max={k_max} tau={tau}")
        res = _run_commit_match(st, parent, V, 0.0, 8, 8, 0, lg, S_max=-1, k_max=k_max, tau=tau)
        check_commit_match(dict(state=st, parent=parent), res, 0.0, 8, 8, 0, -1, logits_host=lg,
                           k_max=k_max, tau=tau)
        if k_max == 3:
            assert list(res["commit_pos"][0]) == [2, 4, 5]
    assert np.all(res["next_state"] != -1)


@pytest.mark.parametrize("case", range(3))
def test_threshold_planted_chain(gpu_lib, case):
    """Drafts that each add up to k_max positions (the target's own threshold
    commits) are matched hop by hop."""
    rng = np.random.default_rng(700 + case)
    N, V, seed, k_max = [16, 32, 64][case], [2048, 4096, 151936][case], 5 + case, [2, 3, 4][case]
    T, tau = [0.0, 1.0, 0.7][case], [0.0, 1e-3, 0.5][case]
    depth = int(rng.integers(2, 5))
    st, parent, planted = _planted_case(rng, N, V, T, 40, 512, seed, depth, decoys=8,
                                        k_max=k_max, tau=tau)
    say(f"threshold planted case {case} B1={st.shape[0]} N={N} k_max={k_max} tau={tau} depth={depth}")
    rows = O.masked_rows(st)
    lg = np.stack([synth.state_keyed_logits(seed, st[r // N], V)[r % N] for r in rows])
    res = _run_commit_match(st, parent, V, T, seed, 40, 512, lg, S_max=k_max, k_max=k_max, tau=tau)
    h = check_commit_match(dict(state=st, parent=parent), res, T, seed, 40, 512, k_max,
                           logits_host=lg, k_max=k_max, tau=tau)
    assert h == planted


@pytest.mark.parametrize("idx", [2, 3])
def test_threshold_commit_workload(gpu_lib, idx):
    """Threshold commit at the full workload shape on seeded host logits."""
    wl = synth.WORKLOADS[idx]
    x = host_inputs(idx)
    xd = to_device(x)
    step = step_for(wl, x, k_max=4, tau=0.0)
    step.masked_rows(xd)
    lg = synth.draw_logits(step.M, wl.V, wl.seed + 1000)
    rows = O.masked_rows(x["state"])
    *_, conf, _S = O.commit(lg, rows, x["state"], x["parent"], wl.T, wl.seed, wl.step0, wl.pos0)
    for q in (0.0, 0.5, 0.9):
        tau = float(np.quantile(conf, q))
        step.tau = tau
        say(f"workload {idx} threshold commit k_max=4 tau={tau:.4g}")
        res = commit_on(step, xd, lg)
        check_commit_match(x, res, wl.T, wl.seed, wl.step0, wl.pos0, wl.S_t, logits_host=lg,
                           k_max=4, tau=tau)
    del xd, step
    torch.cuda.empty_cache()
