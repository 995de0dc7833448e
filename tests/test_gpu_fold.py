"""GPU parity of SpecFold folded verification against the CPU oracle, through
the C ABI: gate flags, sources and compacted lists bit-exact; folded attention
within the dense attention's tolerances of the oracle's definition (attention
of the resolved query over the branch's resolved table); delta < 0 agrees
with the dense kernel."""
import functools
import sys

import numpy as np
import pytest
import torch

from branch_verify_amd import synth
from branch_verify_amd.step import FoldedAttention, VerifyStep, folded_for, to_device
from oracle import fold as F
from oracle import oracle as O

pytestmark = pytest.mark.gpu

ATT_ABS = 2e-2
LSE_REL = 1e-5
f32 = synth.bf16_bits_to_f32


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def inputs(idx):
    wl = synth.WORKLOADS[idx]
    x = synth.draw_inputs(wl, with_w=False)
    x["h_layer"] = synth.draw_fold_hidden(wl, x["parent"], x["state"])
    return x


def oracle_gate(H_bits, parent, delta):
    Hf = f32(H_bits)
    num, den = F.fold_residual(Hf, parent)
    d32 = float(np.float32(delta))
    if d32 >= 0 and num.shape[0] > 1:
        thr = (d32 * d32) * den[1:]
        gap = np.abs(num[1:] - thr)
        near = gap <= 1e-9 * np.maximum(thr, 1e-300)
        assert not near.any(), "a seeded slot sits on the fold threshold"
    return F.fold_gate(Hf, parent, delta)


def check_lists(fa, ref):
    rec, src, rows, off = ref
    got = fa.lists()
    assert np.array_equal(got["recompute"], rec)
    assert np.array_equal(got["src"], src)
    assert got["count"] == rows.size
    assert np.array_equal(got["rec_rows"], rows)
    assert np.array_equal(got["branch_off"], off)
    pos = np.full(rec.size, -1, np.int64)
    pos[rows] = np.arange(rows.size)
    assert np.array_equal(got["rec_pos"].reshape(-1), pos)


def check_attention(x, fa, src, full, tag):
    o_gpu = fa.o.float().cpu().numpy()
    lse_gpu = fa.lse.cpu().numpy()
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    qr, kr, vr = F.resolve_tables(f32(x["q"]), f32(x["k_blk"]), f32(x["v_blk"]), src)
    kc, vc = f32(x["k_ctx"]), f32(x["v_ctx"])
    if full:
        o_ref, lse_ref = O.attention(qr, kr, vr, kc, vc, fa.scale)
        err_o = np.max(np.abs(o_gpu - o_ref))
        err_l = np.max(np.abs(lse_gpu - lse_ref) / np.abs(lse_ref))
    else:
        rng = np.random.default_rng(0)
        B1, N, Hq = lse_gpu.shape
        G = Hq // fa.Hkv
        samples = [(int(rng.integers(B1)), int(rng.integers(N)), int(rng.integers(Hq))) for _ in range(160)]
        samples += [(0, 0, 0), (B1 - 1, N - 1, Hq - 1)]
        err_o = err_l = 0.0
        for (i, n, h) in samples:
            g = h // G
            o, l = O.attention(qr[i:i + 1, n:n + 1, h:h + 1], kr[i:i + 1, :, g:g + 1], vr[i:i + 1, :, g:g + 1],
                               kc[g:g + 1], vc[g:g + 1], fa.scale)
            err_o = max(err_o, float(np.max(np.abs(o_gpu[i, n, h] - o[0, 0, 0]))))
            err_l = max(err_l, float(abs(lse_gpu[i, n, h] - l[0, 0, 0]) / abs(l[0, 0, 0])))
    say(f"{tag}: folded attention max|dO|={err_o:.3e} max rel dLSE={err_l:.3e}")
    assert err_o <= ATT_ABS
    assert err_l <= LSE_REL


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("delta", [0.1, 0.3])
def test_folded_verification_parity(gpu_lib, idx, delta):
    wl = synth.WORKLOADS[idx]
    x = inputs(idx)
    say(f"folded verification, workload {idx} {wl.name}, delta={delta}")
    ref = oracle_gate(x["h_layer"], x["parent"], delta)
    xd = to_device({k: v for k, v in x.items() if k not in ("parent", "state")})
    fa = folded_for(wl, x["parent"])
    fa.run(xd, xd["h_layer"], delta)
    torch.cuda.synchronize()
    check_lists(fa, ref)
    say(f"workload {idx}: gate exact, fold ratio {F.fold_ratio(ref[0]):.3f}")
    check_attention(x, fa, ref[1], full=idx <= 3, tag=f"workload {idx}")
    # run again: bit-identical
    o1, l1 = fa.o.clone(), fa.lse.clone()
    fa.run(xd, xd["h_layer"], delta)
    torch.cuda.synchronize()
    assert torch.equal(o1, fa.o) and torch.equal(l1, fa.lse)
    del xd, fa
    torch.cuda.empty_cache()


@pytest.mark.parametrize("idx", [2, 3])
def test_nothing_folds_equals_dense_kernel(gpu_lib, idx):
    """delta < 0 recomputes every slot: the folded path computes the dense
    attention (context and block states merged in another order), so it
    agrees with the dense kernel to bf16 rounding of the output."""
    wl = synth.WORKLOADS[idx]
    x = inputs(idx)
    xd = to_device({k: v for k, v in x.items() if k not in ("parent", "state")})
    fa = folded_for(wl, x["parent"])
    fa.run(xd, xd["h_layer"], -1.0)
    dense = VerifyStep(wl.B1, wl.N, wl.L, wl.Hq, wl.Hkv, wl.d, 64, 8, 0, x["parent"], 0.0, 1, 1, 0)
    dense.attend(xd)
    torch.cuda.synchronize()
    lists = fa.lists()
    assert lists["recompute"].all() and lists["count"] == wl.B1 * wl.N
    torch.testing.assert_close(fa.o.float(), dense.o.float(), rtol=0, atol=8e-3)
    torch.testing.assert_close(fa.lse, dense.lse, rtol=2e-6, atol=0)
    check_attention(x, fa, np.arange(wl.B1)[:, None].repeat(wl.N, 1), full=True, tag="delta<0")


def test_everything_folds_copies_main_branch(gpu_lib):
    wl = synth.WORKLOADS[2]
    x = inputs(2)
    xd = to_device({k: v for k, v in x.items() if k not in ("parent", "state")})
    fa = folded_for(wl, x["parent"])
    fa.run(xd, xd["h_layer"], 1e30)
    torch.cuda.synchronize()
    lists = fa.lists()
    assert lists["count"] == wl.N and np.all(lists["src"] == 0)
    for i in range(1, wl.B1):
        torch.testing.assert_close(fa.o[i].float(), fa.o[0].float(), rtol=0, atol=8e-3)
        torch.testing.assert_close(fa.lse[i], fa.lse[0], rtol=1e-6, atol=0)


def _random_case(rng, B1, N, L, Hq, Hkv, d, D, tree):
    if tree == "chain":
        parent = np.array([-1] + list(range(B1 - 1)), np.int32)
    elif tree == "star":
        parent = np.array([-1] + [0] * (B1 - 1), np.int32)
    else:
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, B1)], np.int32)
    H = np.empty((B1, N, D), np.float32)
    H[0] = rng.standard_normal((N, D))
    for i in range(1, B1):
        sig = np.exp(rng.uniform(np.log(0.01), np.log(1.0), (N, 1))).astype(np.float32)
        H[i] = H[parent[i]] + sig * rng.standard_normal((N, D), dtype=np.float32)
        H[i] = f32(synth.f32_to_bf16_bits(H[i]))
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    x = dict(q=bf(B1, N, Hq, d), k_blk=bf(B1, N, Hkv, d), v_blk=bf(B1, N, Hkv, d),
             k_ctx=bf(Hkv, max(L, 1), d)[:, :L], v_ctx=bf(Hkv, max(L, 1), d)[:, :L],
             h_layer=synth.f32_to_bf16_bits(H))
    return parent, x


@pytest.mark.parametrize("shape", [
    dict(B1=12, N=7, L=100, Hq=8, Hkv=1, d=64, D=64, tree="chain"),
    dict(B1=2, N=1, L=0, Hq=2, Hkv=2, d=32, D=8, tree="chain"),
    dict(B1=17, N=40, L=300, Hq=16, Hkv=2, d=128, D=256, tree="random"),
    dict(B1=64, N=3, L=70, Hq=4, Hkv=4, d=128, D=64, tree="random"),
    dict(B1=5, N=256, L=130, Hq=2, Hkv=1, d=32, D=128, tree="star"),
    dict(B1=9, N=32, L=0, Hq=32, Hkv=8, d=128, D=512, tree="chain"),
])
def test_folded_ragged(gpu_lib, shape):
    rng = np.random.default_rng(shape["B1"] * 7 + shape["N"])
    B1, N, L, Hq, Hkv, d, D = (shape[k] for k in ("B1", "N", "L", "Hq", "Hkv", "d", "D"))
    say(f"folded ragged {shape}")
    parent, x = _random_case(rng, B1, N, L, Hq, Hkv, d, D, shape["tree"])
    ref = oracle_gate(x["h_layer"], parent, 0.2)
    xd = to_device(x)
    fa = FoldedAttention(B1, N, L, Hq, Hkv, d, D, parent)
    fa.run(xd, xd["h_layer"], 0.2)
    torch.cuda.synchronize()
    check_lists(fa, ref)
    check_attention(x, fa, ref[1], full=True, tag=f"ragged B1={B1} N={N}")
