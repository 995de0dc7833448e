"""Throughput of one multi-branch verification step on one MI355X.

A step is the whole hot path over one batch: shared-prefix attention of every
branch, masked-row scan, LM head over the masked rows, commit, and the
draft-tree match, with all inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--secondary 2]
                    [--no-cpu-baseline] [--flush-mall]

The headline workload is the largest single-GPU configuration, the
Qwen3-32B-like wide step (33 branches x 64, context 4096, T = 1); the
SDAR-8B-like budget-8 step is timed the same way and reported as a secondary
object of the same line.

value = B1*N branch-tokens verified per step / seconds per step, over K steps
replayed from a HIP graph of one step (the attention runs in order, or on a
second stream beside the commit when it is long).  A second pass of K steps
issued in order on one stream times each call with HIP events on the stream
it runs on; the roofline object reports the dominant kernel (the LM head) from
those against its binding peak (HBM bytes, or bf16 MFMA FLOP when those take
longer), with the HBM traffic its byte counters measured on this workload.
With --flush-mall a 512 MiB buffer is overwritten before every step of that
pass (outside the events), so the per-kernel times start from a cold
last-level cache.  cpu_baseline times the CPU oracle on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified branch-tokens/s per verify step; % HBM peak (attn) and % MFMA peak (LM head)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
MALL_FLUSH_BYTES = 512 << 20   # twice the 256 MB last-level cache


def note(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--secondary", type=int, default=2,
                    help="a second workload timed the same way (graph replay and per-kernel events) "
                         "and reported inside the line; 0 for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mall", action="store_true",
                    help="overwrite a 512 MiB buffer before every step of the per-kernel event pass")
    ap.add_argument("--no-side-legs", action="store_true",
                    help="time only the step (no threshold, folded, drafting or tray legs)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the attention in order on the main stream whatever --attn-with says")
    ap.add_argument("--attn-with", choices=["auto", "in_order", "commit", "lm_head"], default="auto",
                    help="run the attention first in order, or on a second stream beside the commit "
                         "or beside the LM head; auto: in order unless it is long, then beside the commit")
    ap.add_argument("--no-graph", action="store_true",
                    help="issue the timed steps call by call instead of replaying a HIP graph")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before the steps, run 3 plain device copies of this many bytes "
                         "(the calibration kernel for the HBM byte counters)")
    ap.add_argument("--cpu-only", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


def algorithmic(wl, M):
    """Bytes and flops each kernel must move/compute (context K/V read once)."""
    B1, N, L, Hq, Hkv, d, D, V = wl.B1, wl.N, wl.L, wl.Hq, wl.Hkv, wl.d, wl.D, wl.V
    R = B1 * N
    attn_bytes = 2 * (R * Hq * d * 2 + 2 * R * Hkv * d + 2 * Hkv * L * d) + 4 * R * Hq
    attn_flop = 4 * R * Hq * d * (L + N)
    lm_bytes = 2 * V * D + 2 * M * D + 4 * M * V + 4 * M
    lm_flop = 2 * M * D * V
    commit_bytes = 4 * M * V + 4 * 2 * R + 8 * M
    return dict(attention=(attn_bytes, attn_flop), lm_head=(lm_bytes, lm_flop),
                commit=(commit_bytes, 0))


LM_HEAD_SOURCES = [os.path.join(ROOT, "branch_verify_amd", "csrc", f) for f in ("lm_head.hip", "common.h")]


def source_digest(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per LM-head launch from a committed counter summary
    (profiles/lm_head_*_counters.md) taken on this workload, or None when
    there is none or the kernel source changed since the counters were taken."""
    here = source_digest(LM_HEAD_SOURCES)
    for name in sorted(os.listdir(PROFILES)):
        if not (name.startswith("lm_head_") and name.endswith("_counters.md")):
            continue
        text = open(os.path.join(PROFILES, name)).read()
        m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
        s = re.search(r"lm_head_source_sha256_16:\s*([0-9a-f]+)", text)
        w = re.search(r"traffic_workload:\s*(\S+)", text)
        if m and s and w and w.group(1) == workload and s.group(1) == here:
            return float(m.group(1))
    return None


def _oracle_steps(wl, x, budget_s, max_steps):
    """Full oracle steps of one workload until about budget_s seconds of CPU
    work; returns the per-step wall times."""
    import numpy as np

    from branch_verify_amd import synth
    from oracle import oracle as O
    f = synth.bf16_bits_to_f32
    args = [f(x[k]) for k in ("q", "k_blk", "v_blk", "k_ctx", "v_ctx", "hidden")]
    w = f(x["w"])
    times = []
    while len(times) < max_steps and (not times or sum(times) < budget_s):
        t0 = time.perf_counter()
        O.verify_step(*args, w, x["state"], x["parent"], wl.T, wl.seed, wl.step0, wl.pos0,
                      1.0 / np.sqrt(wl.d), S_max=wl.S_t)
        times.append(time.perf_counter() - t0)
    return times


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, single_wl=None, single_x=None):
    """The CPU oracle over the same workload (full steps, about 10-30 s of CPU
    work), with numpy's BLAS on every core this process may use; and, when
    single_wl is given, one full step of that (smaller) workload with BLAS
    limited to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] + [1])
    blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer', '?')})"
                     for p in pools if p.get("user_api") == "blas") or "none found"
    times = _oracle_steps(wl, x, 10.0, 10)
    dt = float(np.median(times))
    out = {"value": wl.B1 * wl.N / dt, "unit": "branch-tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{len(times)} full verify step(s) of {wl.name} (fp64 numpy oracle: attention, "
                     f"LM head, commit, match), median {dt:.2f} s per step",
           "cpu_model": _cpu_model(), "blas": blas,
           "affinity_cores": len(os.sched_getaffinity(0))}
    if single_wl is not None:
        with threadpool_limits(limits=1):
            t1 = _oracle_steps(single_wl, single_x, 0.0, 1)
        out["single_thread"] = {"workload": single_wl.name, "value": single_wl.B1 * single_wl.N / t1[0],
                                "unit": "branch-tokens/s", "cores": 1, "s_per_step": t1[0]}
    return out


def measure_step(wl, x, a, note_prefix=""):
    """Warm-up, the timed graph replays, and the per-kernel event pass of one
    workload's step.  Returns (step, device inputs, timing dict)."""
    import numpy as np
    import torch

    from branch_verify_amd.step import step_for, to_device

    xd = to_device(x)
    step = step_for(wl, x)
    stream = torch.cuda.current_stream()
    note(f"{note_prefix}{a.warmup} warm-up steps, then {a.steps} timed steps")
    for _ in range(a.warmup):
        step.run(xd)
    torch.cuda.synchronize()

    # Timed region: K whole steps (the attention in order, or on a second
    # stream joined inside each step, as --attn-with places it), replayed from
    # a HIP graph of one step unless --no-graph, bracketed by synchronize.
    if not a.no_graph:
        step.capture(xd, overlap=not a.no_overlap, attn_with=a.attn_with)
        for _ in range(2):
            step.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        if a.no_graph:
            step.run(xd, overlap=not a.no_overlap, attn_with=a.attn_with)
        else:
            step.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-kernel times: K more steps issued in order on one stream, with HIP
    # events around each call on the stream it is launched on.
    names = ["attention", "masked_rows", "lm_head", "commit", "match"]
    calls = [step.attend, step.masked_rows, step.head, step.commit_step, step.match]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in names] for _ in range(a.steps)]
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device="cuda") if a.flush_mall else None
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(a.steps):
        if flush is not None:
            flush.fill_(s & 0xFF)
        for j, fn in enumerate(calls):
            ev[s][j][0].record(stream)
            fn(xd)
            ev[s][j][1].record(stream)
    torch.cuda.synchronize()
    elapsed_seq = time.perf_counter() - t1
    del flush
    per = {n: float(np.mean([ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(a.steps)])) * 1e3
           for j, n in enumerate(names)}  # microseconds
    M = step.M
    alg = algorithmic(wl, M)
    lm_bytes, lm_flop = alg["lm_head"]
    lm_s = per["lm_head"] * 1e-6
    # the LM head's binding roofline: HBM bytes or bf16 MFMA FLOP, whichever
    # takes longer at its peak
    mfma_bound = lm_flop / (BF16_PEAK_TFLOPS * 1e12) > lm_bytes / (HBM_PEAK_GBS * 1e9)
    achieved = lm_flop / lm_s / 1e12 if mfma_bound else lm_bytes / lm_s / 1e9
    out = {
        "value": wl.B1 * wl.N / (elapsed / a.steps),
        "ms_per_step": elapsed / a.steps * 1e3,
        "config": {"workload": wl.name, "B1": wl.B1, "N": wl.N, "L": wl.L, "Hq": wl.Hq,
                   "Hkv": wl.Hkv, "d": wl.d, "D": wl.D, "V": wl.V, "masked_rows": M,
                   "temperature": wl.T, "parallelism": "none (1 GPU)",
                   "launch": "call by call" if a.no_graph else "hip graph",
                   "attention": "in order" if a.no_overlap else
                   {"in_order": "in order", "commit": "beside the commit",
                    "lm_head": "beside the LM head"}[step.attn_placement(a.attn_with)],
                   "per_kernel_cache": "cold (512 MiB overwritten before each step)" if a.flush_mall
                   else "warm"},
        "roofline": {"bound": "mfma" if mfma_bound else "hbm", "kernel": "lm_head",
                     "achieved": achieved,
                     "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": achieved / (BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS),
                     "traffic": measured_traffic(wl.name),
                     "algorithmic_bytes": lm_bytes, "algorithmic_flop": lm_flop,
                     "hbm_frac": lm_bytes / lm_s / 1e9 / HBM_PEAK_GBS,
                     "mfma_frac": lm_flop / lm_s / 1e12 / BF16_PEAK_TFLOPS},
        "kernels_us": per,
        "ms_per_step_sequential": elapsed_seq / a.steps * 1e3,
    }
    ab, af = alg["attention"]
    out["attention_roofline"] = {"hbm_frac": ab / (per["attention"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                 "mfma_frac": af / (per["attention"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
    cb, _ = alg["commit"]
    if step.fuse:  # the commit reads the LM head's tile partials, not the logits
        cb = cb - 4 * M * wl.V + step.parts_bytes
    out["commit_roofline"] = {"hbm_frac": cb / (per["commit"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "reads": "tile partials" if step.fuse else "logits"}
    return step, xd, out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the step is not "
              "sharded across GPUs", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from branch_verify_amd import synth
    from branch_verify_amd.step import step_for, to_device

    wl = synth.WORKLOADS[a.workload]
    sec_wl = synth.WORKLOADS[a.secondary] if a.secondary and a.secondary != a.workload else None
    note(f"drawing inputs of {wl.name}")
    x = synth.draw_inputs(wl)
    M = synth.masked_count(x["state"])
    if a.cpu_only:
        sx = synth.draw_inputs(sec_wl) if sec_wl is not None else None
        print(json.dumps(cpu_baseline(wl, x, sec_wl, sx)))
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stream = torch.cuda.current_stream()

    if a.copy_bytes > 0:
        note(f"calibration: 3 device copies of {a.copy_bytes} bytes")
        src = torch.empty(a.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the secondary workload first, then the headline one (whose buffers the
    # side legs below reuse)
    secondary, sx = None, None
    if sec_wl is not None:
        note(f"secondary workload {sec_wl.name}")
        sx = synth.draw_inputs(sec_wl)
        s_step, s_xd, secondary = measure_step(sec_wl, sx, a, note_prefix=f"{sec_wl.name}: ")
        del s_step, s_xd
        torch.cuda.empty_cache()

    step, xd, head = measure_step(wl, x, a, note_prefix=f"{wl.name}: ")
    per = head["kernels_us"]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "branch-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    out.update({k: v for k, v in head.items() if k not in ("value", "ms_per_step")})
    if secondary is not None:
        out["secondary"] = secondary
    if a.no_side_legs:
        if not a.no_cpu_baseline:
            note("timing the CPU oracle")
        out["cpu_baseline"] = None if a.no_cpu_baseline else cpu_baseline(wl, x, sec_wl, sx)
        print(json.dumps(out))
        return
    cb, _ = algorithmic(wl, M)["commit"]
    if step.fuse:  # the commit reads the LM head's tile partials, not the logits
        cb = cb - 4 * M * wl.V + step.parts_bytes

    # The threshold variant of the commit (up to k_max positions with
    # confidence >= 0.9 per branch), on the same logits, timed the same way.
    # (The side legs report the median call: a single stalled call, seen once
    # at 33 ms, would otherwise dominate a mean of short calls.)
    k_thr, tau_thr = max(2, wl.S_t), 0.9
    thr = step_for(wl, x, k_max=k_thr, tau=tau_thr, fuse=False)
    thr.masked_rows(xd)
    tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    for _ in range(max(1, a.warmup)):  # (its kernels' first launch loads their code)
        thr.commit(xd, logits=step.logits)
    for s in range(a.steps):
        tev[s][0].record(stream)
        thr.commit(xd, logits=step.logits)
        tev[s][1].record(stream)
    torch.cuda.synchronize()
    thr_us = float(np.median([b.elapsed_time(e) for b, e in tev])) * 1e3
    thr_taken = int((thr.commit_pos >= 0).sum().item())
    del thr

    # SpecFold folded verification of the same batch's attention (delta 0.1):
    # the gate on synthetic layer-input hidden states, then recomputed rows
    # plus corrected folded rows; timed the same way as the dense attention.
    from branch_verify_amd.step import folded_for
    fold_delta = 0.1
    h_layer = to_device({"h": synth.draw_fold_hidden(wl, x["parent"], x["state"])})["h"]
    fa = folded_for(wl, x["parent"])
    for _ in range(3):
        fa.run(xd, h_layer, fold_delta)
    torch.cuda.synchronize()
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for s in range(a.steps):
        fev[s][0].record(stream)
        fa.gate(h_layer, fold_delta)
        fev[s][1].record(stream)
        fa.attend(xd)
        fev[s][2].record(stream)
    torch.cuda.synchronize()
    gate_us = float(np.median([e[0].elapsed_time(e[1]) for e in fev])) * 1e3
    fattn_us = float(np.median([e[1].elapsed_time(e[2]) for e in fev])) * 1e3
    rec = fa.lists()["recompute"]
    fold_ratio = float(1.0 - rec[1:].mean()) if wl.B1 > 1 else 0.0
    gate_bytes = 2 * 2 * (wl.B1 - 1) * wl.N * wl.D + 4 * 5 * wl.B1 * wl.N
    del fa, h_layer

    # Drafting the next tree from this pass's stale conditionals of the main
    # branch: top-32 per masked position, then a best-first tree of B1-1
    # drafts with 4 children per node.
    from branch_verify_amd import sfv
    K_top, D_tree, W_tree = 32, wl.B1 - 1, 4
    top_ids = torch.zeros((wl.N, K_top), dtype=torch.int32, device="cuda")
    top_val = torch.zeros((wl.N, K_top), dtype=torch.float32, device="cuda")
    conf_pos = torch.zeros((wl.N,), dtype=torch.float32, device="cuda")
    t_par = torch.zeros((D_tree + 1,), dtype=torch.int32, device="cuda")
    t_st = torch.zeros((D_tree + 1, wl.N), dtype=torch.int32, device="cuda")
    t_nd = torch.zeros((1,), dtype=torch.int32, device="cuda")
    root = xd["state"][0]

    topk_wsb = sfv.sfv_stale_topk_workspace_bytes(step.M, wl.V, wl.N, K_top)
    topk_ws = torch.empty(max(topk_wsb, 16), dtype=torch.uint8, device="cuda")

    def draft_once():
        sfv.sfv_stale_topk(step.logits, step.rows, step.conf, step.M, wl.V, wl.N, 0, K_top, top_ids, top_val,
                           conf_pos, topk_ws, topk_wsb)
        dev[1].record(stream)
        sfv.sfv_draft_tree(root, top_ids, top_val, conf_pos, wl.N, K_top, D_tree, W_tree, wl.T, wl.seed,
                           wl.step0 + 1, wl.pos0, t_par, t_st, t_nd)

    dev = [None, torch.cuda.Event(enable_timing=True)]
    for _ in range(3):
        draft_once()
    torch.cuda.synchronize()
    dtimes = []
    for s_ in range(a.steps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        dev[1] = e1
        e0.record(stream)
        draft_once()
        e2.record(stream)
        dtimes.append((e0, e1, e2))
    torch.cuda.synchronize()
    topk_us = float(np.median([e0.elapsed_time(e1) for e0, e1, _ in dtimes])) * 1e3
    tree_us = float(np.median([e1.elapsed_time(e2) for _, e1, e2 in dtimes])) * 1e3
    main_rows = int((x["state"][0] == -1).sum())
    n_drafted = int(t_nd.item())
    del topk_ws

    # Packed-tray verification for an autoregressive target (24 trays of 16
    # drafted tokens, the packed budget of 384): causal tray attention over
    # this workload's context and heads, then rejection sampling on seeded
    # target logits and proposals of the same shape.
    n_tr, B_tr = 24, 16
    tr_logits, tr_q, tr_tok = synth.draw_trays(n_tr, B_tr, wl.V, seed=wl.seed + 500, T=1.0, drift=0.6)
    tl, tq, tt = (torch.from_numpy(v).cuda() for v in (tr_logits, tr_q, tr_tok))
    del tr_logits, tr_q
    tr_na = torch.zeros(n_tr, dtype=torch.int32, device="cuda")
    tr_nt = torch.zeros(n_tr, dtype=torch.int32, device="cuda")
    rj_wsb = sfv.sfv_reject_workspace_bytes(n_tr, B_tr, wl.V)
    rj_ws = torch.empty(rj_wsb, dtype=torch.uint8, device="cuda")
    rng_t = np.random.default_rng(wl.seed + 501)
    tq_bits = lambda *sh: torch.from_numpy(
        synth.f32_to_bf16_bits(rng_t.standard_normal(sh, dtype=np.float32))).view(torch.bfloat16).cuda()
    ta_q = tq_bits(n_tr, B_tr, wl.Hq, wl.d)
    ta_k = tq_bits(n_tr, B_tr, wl.Hkv, wl.d)
    ta_v = tq_bits(n_tr, B_tr, wl.Hkv, wl.d)
    ta_o = torch.empty((n_tr, B_tr, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda")
    ta_lse = torch.empty((n_tr, B_tr, wl.Hq), dtype=torch.float32, device="cuda")
    ta_wsb = sfv.sfv_attend_workspace_bytes(n_tr, B_tr, wl.L, wl.Hq, wl.Hkv, wl.d)
    ta_ws = torch.empty(max(ta_wsb, 16), dtype=torch.uint8, device="cuda")

    def trays_once(ev=None):
        sfv.sfv_attend_trays(ta_q, ta_k, ta_v, xd["k_ctx"], xd["v_ctx"], n_tr, B_tr, wl.L, wl.Hq, wl.Hkv, wl.d,
                             1.0 / np.sqrt(wl.d), ta_o, ta_lse, ta_ws, ta_wsb)
        if ev is not None:
            ev.record(stream)
        sfv.sfv_reject_verify(tl, tq, tt, n_tr, B_tr, wl.V, 1.0, wl.seed, wl.step0, wl.pos0, tr_na, tr_nt,
                              rj_ws, rj_wsb)

    for _ in range(2):
        trays_once()
    torch.cuda.synchronize()
    ttimes = []
    for s_ in range(a.steps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        trays_once(e1)
        e2.record(stream)
        ttimes.append((e0, e1, e2))
    torch.cuda.synchronize()
    tray_attn_us = float(np.median([e0.elapsed_time(e1) for e0, e1, _ in ttimes])) * 1e3
    reject_us = float(np.median([e1.elapsed_time(e2) for _, e1, e2 in ttimes])) * 1e3
    tray_accepted = tr_na.cpu().numpy()
    reject_bytes = 2 * 4 * n_tr * (B_tr + 1) * wl.V + 4 * n_tr * wl.V * 2   # two passes per row + emitting rows
    del tl, tq, tt, rj_ws, ta_q, ta_k, ta_v, ta_o, ta_lse, ta_ws
    out["folded_attention"] = {"delta": fold_delta, "fold_ratio": fold_ratio, "gate_us": gate_us,
                               "attention_us": fattn_us, "dense_attention_us": per["attention"],
                               "speedup_vs_dense": per["attention"] / (gate_us + fattn_us),
                               "gate_hbm_frac": gate_bytes / (gate_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    out["drafting"] = {"K": K_top, "D": D_tree, "W": W_tree, "topk_us": topk_us, "tree_us": tree_us,
                       "main_masked_rows": main_rows, "drafts_built": n_drafted,
                       "topk_hbm_frac": 2 * 4 * main_rows * wl.V / (topk_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    out["tray_verify"] = {"n_trays": n_tr, "B": B_tr, "temperature": 1.0, "attention_us": tray_attn_us,
                          "reject_us": reject_us, "mean_accepted": float(tray_accepted.mean()),
                          "reject_hbm_frac": reject_bytes / (reject_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    out["commit_threshold"] = {"k_max": k_thr, "tau": tau_thr, "us": thr_us,
                               "positions_committed": thr_taken,
                               "hbm_frac": cb / (thr_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    if not a.no_cpu_baseline:
        note("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(wl, x, sec_wl, sx)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
