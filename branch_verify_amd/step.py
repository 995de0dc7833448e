"""One verification step on the GPU through the C ABI.

PyTorch provides device memory and the stream; the five calls below do all of
the work in libsfv's kernels: shared-prefix attention, masked-row scan, LM head
over the masked rows, commit, and the draft-tree match.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import sfv

# Attention work (4 * rows * query heads * d * keys) from which the automatic
# placement overlaps it with the commit instead of running it in order.
ATTN_OVERLAP_FLOP = 50e9


def to_device(inp: dict, device="cuda") -> dict:
    """Host inputs from synth.draw_inputs -> device tensors (bf16 stays bf16)."""
    out = {}
    for k, v in inp.items():
        if k == "parent":
            out[k] = np.asarray(v, dtype=np.int32)
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        out[k] = t.to(device)
    return out


class VerifyStep:
    """Buffers and calls of one multi-branch verification step of fixed shape."""

    def __init__(self, B1, N, L, Hq, Hkv, d, D, V, M, parent, temperature, seed, step0, pos0,
                 S_max=-1, k_max=1, tau=0.0, fuse=True, device="cuda"):
        sfv.load()
        self.B1, self.N, self.L, self.Hq, self.Hkv, self.d = B1, N, L, Hq, Hkv, d
        self.D, self.V, self.M = D, V, M
        self.parent = [int(x) for x in parent]
        self.T, self.seed, self.step0, self.pos0 = float(temperature), seed, step0, pos0
        self.S_max = S_max
        self.k_max, self.tau = int(k_max), float(tau)
        self.scale = 1.0 / math.sqrt(d)
        dev = device
        self.o = torch.empty((B1, N, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B1, N, Hq), dtype=torch.float32, device=dev)
        self.attn_ws_bytes = sfv.sfv_attend_workspace_bytes(B1, N, L, Hq, Hkv, d)
        self.attn_ws = torch.empty(max(1, self.attn_ws_bytes), dtype=torch.uint8, device=dev)
        self.rows = torch.zeros(B1 * N, dtype=torch.int32, device=dev)
        self.count = torch.empty(1, dtype=torch.int32, device=dev)
        self.logits = torch.empty((max(1, M), V), dtype=torch.float32, device=dev)
        self.commit_ws_bytes = sfv.sfv_commit_workspace_bytes(B1, N, M, V)
        self.commit_ws = torch.empty(max(1, self.commit_ws_bytes), dtype=torch.uint8, device=dev)
        # greedy steps from 33 rows on: the LM head writes tile partials and
        # the commit reads those instead of the logits
        self.parts_bytes = sfv.sfv_lm_head_greedy_bytes(M, V, D) if (fuse and self.T == 0.0) else 0
        self.fuse = self.parts_bytes > 0
        if self.fuse:
            self.parts = torch.empty(self.parts_bytes, dtype=torch.uint8, device=dev)
            self.greedy_ws_bytes = sfv.sfv_commit_greedy_workspace_bytes(B1, N, M, V)
            self.greedy_ws = torch.empty(max(1, self.greedy_ws_bytes), dtype=torch.uint8, device=dev)
        self.next_state = torch.empty((B1, N), dtype=torch.int32, device=dev)
        self.commit_pos = torch.empty((B1, self.k_max), dtype=torch.int32, device=dev)
        self.token = torch.empty(max(1, M), dtype=torch.int32, device=dev)
        self.conf = torch.empty(max(1, M), dtype=torch.float32, device=dev)
        self.chain = torch.empty(B1, dtype=torch.int32, device=dev)
        self.n_accepted = torch.empty(1, dtype=torch.int32, device=dev)
        self.status = torch.empty(1, dtype=torch.int32, device=dev)
        self._side = None  # second stream for the attention (created on first overlapped run)
        self._graph = None

    # the individual rows of the hot path -----------------------------------
    def attend(self, x, stream=None):
        sfv.sfv_attend_branches(x["q"], x["k_blk"], x["v_blk"], x["k_ctx"], x["v_ctx"], self.B1,
                                self.N, self.L, self.Hq, self.Hkv, self.d, self.scale, self.o,
                                self.lse, self.attn_ws, self.attn_ws_bytes, stream)

    def masked_rows(self, x, stream=None):
        sfv.sfv_masked_rows(x["state"], self.B1, self.N, self.rows, self.count, stream)

    def lm_head(self, x, stream=None):
        sfv.sfv_lm_head(x["hidden"], self.rows, self.M, self.B1 * self.N, x["w"], self.D, self.V,
                        self.logits, stream)

    def commit(self, x, logits=None, stream=None):
        sfv.sfv_commit(self.logits if logits is None else logits, self.rows, self.M, x["state"],
                       self.parent, self.B1, self.N, self.V, self.T, self.seed, self.step0,
                       self.pos0, self.k_max, self.tau, self.next_state, self.commit_pos, self.token, self.conf,
                       self.commit_ws, self.commit_ws_bytes, stream)

    def lm_head_greedy(self, x, stream=None):
        sfv.sfv_lm_head_greedy(x["hidden"], self.rows, self.M, self.B1 * self.N, x["w"], self.D, self.V,
                               self.logits, self.parts, self.parts_bytes, stream)

    def commit_greedy(self, x, stream=None):
        sfv.sfv_commit_greedy(self.parts, self.parts_bytes, self.D, self.logits, self.rows, self.M, x["state"],
                              self.parent, self.B1, self.N, self.V, self.k_max, self.tau, self.next_state,
                              self.commit_pos, self.token, self.conf, self.greedy_ws, self.greedy_ws_bytes,
                              stream)

    def head(self, x, stream=None):
        """The LM head of the step (with tile partials when fused)."""
        (self.lm_head_greedy if self.fuse else self.lm_head)(x, stream)

    def commit_step(self, x, stream=None):
        """The commit of the step (from the tile partials when fused)."""
        if self.fuse:
            self.commit_greedy(x, stream)
        else:
            self.commit(x, stream=stream)

    def match(self, x, stream=None):
        sfv.sfv_match_tree(x["state"], self.next_state, self.commit_pos, self.parent, self.B1,
                           self.N, self.k_max, self.S_max, self.chain, self.n_accepted, self.status, stream)

    def attn_placement(self, attn_with="auto"):
        """Where the attention runs: "in_order" (first, on the caller's
        stream), "lm_head" (on a second stream, beside the LM head) or
        "commit" (on a second stream once the LM head is done, beside the
        commit and the walk).

        Two workgroups of the attention fill a CU's registers, so a kernel on
        the other stream shares the GPU with it only CU by CU: overlapping
        pays where one of them leaves CUs idle, not otherwise.  "auto" runs a
        short attention in order and overlaps one of at least
        ATTN_OVERLAP_FLOP with the commit: the last round of its many
        long-lived workgroups leaves most CUs idle, and the commit's sweep
        fills them.  (Beside the large-tile LM head, which holds most of each
        CU's LDS, the attention would only delay its tiles.)"""
        if attn_with == "auto":
            flop = 4.0 * self.B1 * self.N * self.Hq * self.d * (self.L + self.N)
            return "commit" if flop >= ATTN_OVERLAP_FLOP else "in_order"
        if attn_with not in ("in_order", "lm_head", "commit"):
            raise ValueError(f"attn_with must be 'auto', 'in_order', 'lm_head' or 'commit', not {attn_with!r}")
        return attn_with

    def run(self, x, stream=None, overlap=True, attn_with="auto"):
        """The whole hot path, stream-ordered, no host synchronisation.

        Attention depends only on q/k/v, so with overlap=True it may run on a
        second stream, joined before the call returns; everything else stays
        in order on `stream`.  Where it runs is attn_placement(attn_with);
        overlap=False runs it in order whatever attn_with says.
        Greedy steps in the LM head's tile-partial regime (with fuse) commit
        from the partials."""
        attn_with = self.attn_placement(attn_with)
        if not overlap or attn_with == "in_order":
            self.attend(x, stream)
            self.masked_rows(x, stream)
            self.head(x, stream)
            self.commit_step(x, stream)
            self.match(x, stream)
            return
        main = torch.cuda.current_stream() if stream is None else stream
        if self._side is None:
            self._side = torch.cuda.Stream(device=main.device)
            self._fork = torch.cuda.Event()
            self._join = torch.cuda.Event()
        if attn_with == "lm_head":
            self._fork.record(main)
        self.masked_rows(x, main)
        self.head(x, main)
        if attn_with != "lm_head":
            self._fork.record(main)
        self._side.wait_event(self._fork)
        self.attend(x, self._side)
        self.commit_step(x, main)
        self.match(x, main)
        self._join.record(self._side)
        main.wait_event(self._join)

    def capture(self, x, overlap=True, attn_with="auto"):
        """Capture one whole step (both streams) in a HIP graph; replay() then
        launches it with one call.  The graph holds the current buffers and
        inputs: replays recompute the same step."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            self.run(x, stream=cap, overlap=overlap, attn_with=attn_with)  # warm the side stream outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            self.run(x, stream=cap, overlap=overlap, attn_with=attn_with)
        torch.cuda.synchronize()
        self._graph = g
        return g

    def replay(self):
        self._graph.replay()

    def results(self) -> dict:
        torch.cuda.synchronize()
        M = self.M
        return dict(
            o=self.o, lse=self.lse, rows=self.rows[:M].cpu().numpy(), count=int(self.count.item()),
            logits=self.logits[:M], next_state=self.next_state.cpu().numpy(),
            commit_pos=self.commit_pos.cpu().numpy(), token=self.token[:M].cpu().numpy(),
            conf=self.conf[:M].cpu().numpy(), chain=self.chain.cpu().numpy(),
            h=int(self.n_accepted.item()), status=int(self.status.item()))


def step_for(wl, inp: dict, device="cuda", S_max=None, k_max=1, tau=0.0, fuse=True) -> VerifyStep:
    from .synth import masked_count
    M = masked_count(inp["state"])
    return VerifyStep(wl.B1, wl.N, wl.L, wl.Hq, wl.Hkv, wl.d, wl.D, wl.V, M, inp["parent"], wl.T,
                      wl.seed, wl.step0, wl.pos0, S_max=wl.S_t if S_max is None else S_max,
                      k_max=k_max, tau=tau, fuse=fuse, device=device)


class FoldedAttention:
    """SpecFold folded verification of the attention rows of one branch batch:
    the parent-child gate on the layer-input hidden states, then attention
    with recomputed rows computed and folded rows corrected from their source.
    Buffers are allocated once per shape; both calls are stream-ordered."""

    def __init__(self, B1, N, L, Hq, Hkv, d, D, parent, device="cuda"):
        sfv.load()
        self.B1, self.N, self.L, self.Hq, self.Hkv, self.d, self.D = B1, N, L, Hq, Hkv, d, D
        self.parent = [int(x) for x in parent]
        self.scale = 1.0 / math.sqrt(d)
        dev = device
        i32 = dict(dtype=torch.int32, device=dev)
        self.recompute = torch.empty((B1, N), **i32)
        self.src = torch.empty((B1, N), **i32)
        self.rec_rows = torch.empty(B1 * N, **i32)
        self.rec_count = torch.empty(1, **i32)
        self.rec_pos = torch.empty((B1, N), **i32)
        self.branch_off = torch.empty(B1 + 1, **i32)
        self.o = torch.empty((B1, N, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B1, N, Hq), dtype=torch.float32, device=dev)
        self.ws_bytes = sfv.sfv_attend_folded_workspace_bytes(B1, N, L, Hq, Hkv, d)
        self.ws = torch.empty(max(1, self.ws_bytes), dtype=torch.uint8, device=dev)

    def gate(self, h_layer, delta, stream=None):
        sfv.sfv_fold_gate(h_layer, self.parent, self.B1, self.N, self.D, delta, self.recompute,
                          self.src, self.rec_rows, self.rec_count, self.rec_pos, self.branch_off,
                          stream)

    def attend(self, x, stream=None):
        sfv.sfv_attend_folded(x["q"], x["k_blk"], x["v_blk"], x["k_ctx"], x["v_ctx"], self.B1,
                              self.N, self.L, self.Hq, self.Hkv, self.d, self.scale, self.src,
                              self.rec_rows, self.rec_count, self.rec_pos, self.o, self.lse,
                              self.ws, self.ws_bytes, stream)

    def run(self, x, h_layer, delta, stream=None):
        self.gate(h_layer, delta, stream)
        self.attend(x, stream)

    def lists(self) -> dict:
        torch.cuda.synchronize()
        cnt = int(self.rec_count.item())
        return dict(recompute=self.recompute.cpu().numpy().astype(bool), src=self.src.cpu().numpy(),
                    rec_rows=self.rec_rows[:cnt].cpu().numpy(), count=cnt,
                    rec_pos=self.rec_pos.cpu().numpy(), branch_off=self.branch_off.cpu().numpy())


def folded_for(wl, parent, device="cuda") -> FoldedAttention:
    return FoldedAttention(wl.B1, wl.N, wl.L, wl.Hq, wl.Hkv, wl.d, wl.D, parent, device=device)
