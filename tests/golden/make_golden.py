"""Writes tests/golden/tiny_step.json: the oracle's outputs for the tiny
workload (3 branches in a chain, N 8, L 64, 4/2 heads, d 32, D 128, V 512,
greedy).  Calls only the oracle and the seeded input generator."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from branch_verify_amd import synth  # noqa: E402
from oracle import oracle as O      # noqa: E402


def tiny_step():
    wl = synth.WORKLOADS[1]
    x = synth.draw_inputs(wl)
    f = synth.bf16_bits_to_f32
    out = O.verify_step(f(x["q"]), f(x["k_blk"]), f(x["v_blk"]), f(x["k_ctx"]), f(x["v_ctx"]),
                        f(x["hidden"]), f(x["w"]), x["state"], x["parent"], wl.T, wl.seed,
                        wl.step0, wl.pos0, 1.0 / np.sqrt(wl.d), S_max=wl.S_t)
    return {
        "workload": wl.name,
        "parent": [int(v) for v in x["parent"]],
        "state": x["state"].tolist(),
        "rows": [int(v) for v in out["rows"]],
        "token": [int(v) for v in out["token"]],
        "commit_pos": out["commit_pos"][:, 0].tolist(),
        "next_state": out["next_state"].tolist(),
        "chain": [int(v) for v in out["chain"]],
        "h": int(out["h"]),
        "lse_head": [float(v) for v in out["lse"].reshape(-1)[:16]],
        "o_sum": float(out["o"].sum()),
        "logits_sum": float(out["logits"].astype(np.float64).sum()),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_step.json"), "w") as fh:
        json.dump(tiny_step(), fh, indent=1)
