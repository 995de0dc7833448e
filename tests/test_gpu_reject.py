"""GPU parity of rejection-sampling verification of drafted trays and of the
causal tray attention against the CPU oracle, through the C ABI: accepted
counts and emitted tokens bit-exact on the same seeded blocks (decisions
checked to sit away from their thresholds on the oracle side); tray matching
exact; tray attention within the dense attention's tolerances."""
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import sfv, synth
from oracle import oracle as O
from oracle import reject as R

pytestmark = pytest.mark.gpu
f32 = synth.bf16_bits_to_f32


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_reject(logits, q, tokens, T, seed, step0, pos0):
    n, B1, V = logits.shape
    B = B1 - 1
    na = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    nt = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    wsb = sfv.sfv_reject_workspace_bytes(n, B, V)
    ws = torch.empty(wsb + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    wsv = ws[off:off + wsb]
    sfv.sfv_reject_verify(_dev(logits), _dev(q), _dev(tokens.astype(np.int32)), n, B, V, T, seed, step0, pos0,
                          na, nt, wsv, wsb)
    torch.cuda.synchronize()
    return na.cpu().numpy(), nt.cpu().numpy()


def _margins_ok(logits, q, tokens, T, seed, step0, pos0):
    """Every acceptance test of the oracle sits away from its threshold (the
    device sums in another order, within 1e-15 relative)."""
    if T == 0.0:
        return True
    for j in range(tokens.shape[0]):
        for t in range(tokens.shape[1]):
            x = int(tokens[j, t])
            p = R.target_probs(logits[j, t], T)[x]
            uq = R.uniform(seed, step0 + j, pos0 + t) * float(q[j, t, x])
            if abs(uq - p) <= 1e-10 * max(p, uq):
                return False
    return True


@pytest.mark.parametrize("n,B,V,T,drift", [
    (4, 16, 4096, 1.0, 0.8), (24, 16, 151936, 1.0, 0.6), (3, 8, 1000, 0.7, 2.0), (5, 4, 64, 2.0, 0.3),
    (6, 16, 4096, 0.0, 0.5), (2, 1, 33, 1.0, 3.0), (64, 3, 512, 1.0, 1.0),
])
def test_reject_verify_parity(gpu_lib, n, B, V, T, drift):
    logits, q, tokens = synth.draw_trays(n, B, V, seed=n * 7 + B, T=T, drift=drift)
    if T == 0.0:  # make some drafted tokens the argmax so that greedy trays get past position 0
        for j in range(n):
            k = j % (B + 1)
            tokens[j, :k] = np.argmax(logits[j, :k], axis=1)
    seed, step0, pos0 = 17, 300, 2048
    assert _margins_ok(logits, q, tokens, T, seed, step0, pos0)
    say(f"reject n={n} B={B} V={V} T={T}")
    a_ref, c_ref = R.verify_trays(logits, q, tokens, T, seed, step0, pos0)
    a, c = run_reject(logits, q, tokens, T, seed, step0, pos0)
    say(f"accepted {a_ref.tolist()[:8]} ...")
    assert np.array_equal(a, a_ref)
    assert np.array_equal(c, c_ref)


def test_reject_all_accepted_and_none_accepted(gpu_lib):
    V, B, n = 2048, 6, 4
    logits = synth.draw_logits(n * (B + 1), V, 5).reshape(n, B + 1, V)
    q = np.stack([[R.target_probs(logits[j, t], 1.0) for t in range(B)] for j in range(n)]).astype(np.float32)
    q *= np.float32(0.999)            # u * q < p everywhere: every token passes
    tokens = np.argmax(q, axis=2).astype(np.int32)
    a_ref, c_ref = R.verify_trays(logits, q, tokens, 1.0, 3, 0, 0)
    a, c = run_reject(logits, q, tokens, 1.0, 3, 0, 0)
    assert np.all(a == B) and np.array_equal(c, c_ref)
    # a proposal that puts its mass where p is tiny: rejected at once
    tokens2 = np.argmin(logits[:, :B], axis=2).astype(np.int32)
    q2 = np.zeros_like(q)
    for j in range(n):
        for t in range(B):
            q2[j, t, tokens2[j, t]] = 1.0
    a_ref, c_ref = R.verify_trays(logits, q2, tokens2, 1.0, 3, 0, 0)
    a, c = run_reject(logits, q2, tokens2, 1.0, 3, 0, 0)
    assert np.array_equal(a, a_ref) and np.array_equal(c, c_ref)
    assert np.all(a == 0)


def test_match_trays(gpu_lib):
    n_acc = _dev(np.array([3, 0, 5], np.int32))
    nxt = _dev(np.array([77, 1, 2], np.int32))
    k = np.array([0, 1, 3, 3, 16, 3], np.int32)
    alt = np.array([77, 77, 70, 77, 5, 77], np.int32)
    served = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    for verified, want in ((0, 3), (1, -1), (2, -1)):
        sfv.sfv_match_trays(n_acc, nxt, verified, _dev(k), _dev(alt), k.size, served)
        torch.cuda.synchronize()
        exp = R.match_tray(int(n_acc[verified]), int(nxt[verified]), k, alt)
        assert int(served.item()) == exp == want
    big_k = np.full(300, 2, np.int32)
    big_alt = np.arange(300, dtype=np.int32)
    sfv.sfv_match_trays(_dev(np.array([2], np.int32)), _dev(np.array([250], np.int32)), 0, _dev(big_k),
                        _dev(big_alt), 300, served)
    torch.cuda.synchronize()
    assert int(served.item()) == 250


@pytest.mark.parametrize("shape", [
    dict(B1=24, N=16, L=2048, Hq=32, Hkv=8, d=128),
    dict(B1=3, N=7, L=0, Hq=4, Hkv=2, d=64),
    dict(B1=5, N=130, L=100, Hq=2, Hkv=1, d=32),
])
def test_tray_attention_parity(gpu_lib, shape):
    rng = np.random.default_rng(shape["N"])
    B1, N, L, Hq, Hkv, d = (shape[k] for k in ("B1", "N", "L", "Hq", "Hkv", "d"))
    say(f"tray attention {shape}")
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    x = dict(q=bf(B1, N, Hq, d), k_blk=bf(B1, N, Hkv, d), v_blk=bf(B1, N, Hkv, d),
             k_ctx=bf(Hkv, max(L, 1), d)[:, :L], v_ctx=bf(Hkv, max(L, 1), d)[:, :L])
    dv = {k: torch.from_numpy(np.ascontiguousarray(v)).view(torch.bfloat16).cuda() for k, v in x.items()}
    o = torch.empty((B1, N, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B1, N, Hq), dtype=torch.float32, device="cuda")
    wsb = sfv.sfv_attend_workspace_bytes(B1, N, L, Hq, Hkv, d)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    scale = 1.0 / np.sqrt(d)
    sfv.sfv_attend_trays(dv["q"], dv["k_blk"], dv["v_blk"], dv["k_ctx"], dv["v_ctx"], B1, N, L, Hq, Hkv, d, scale,
                         o, lse, ws, wsb)
    torch.cuda.synchronize()
    o_ref, lse_ref = R.tray_attention(*(f32(x[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx")), scale)
    err_o = np.max(np.abs(o.float().cpu().numpy() - o_ref))
    err_l = np.max(np.abs(lse.cpu().numpy() - lse_ref) / np.abs(lse_ref))
    say(f"tray attention max|dO|={err_o:.3e} rel dLSE={err_l:.3e}")
    assert err_o <= 2e-2 and err_l <= 1e-5
