"""Seeded synthetic inputs for the multi-branch verification step.

This module only draws inputs.  It holds none of the step's arithmetic (no
attention, no projection, no sampling rule, no matching), so both the HIP path
and the CPU oracle can be fed from it without sharing any of the method.

Shapes follow the multi-branch verification batch of SpecFold ("Folding
Multi-Branch Redundancy for Faster Speculative Decoding in Diffusion Language
Models", introduction, Fig. 1-(b)): B+1 block states of length N, the main
branch at index 0 and drafts whose parent index is smaller than their own,
each draft adding at most S_t unmasked positions over its parent.  Workload
sizes follow the SDAR-8B targets of the SPOT page ("Data and methods",
budgets 8 and 20), and the packed 384-token trays of the D3D explainer
(draft-budget table).

Recipe (every tensor has its own numpy stream, so any subset can be drawn):
  stream [seed, 1]  tree            chain / par(i) ~ U{0..i-1} / star
  stream [seed, 2]  s_i             U{1..S_t} per draft (0 when S_t = 0)
  stream [seed, 3]  states, tokens  main: m0 masked positions chosen uniformly;
                                    draft: parent + s_i of the parent's masked
                                    positions, tokens U{0..V-1}
  streams [seed, 10..15]  q, k_blk, v_blk, k_ctx, v_ctx, hidden   N(0, 1)
  streams [seed, 16, c]   W rows in chunks of 4096                N(0, w_std)
  streams [seed, 17, 18]  layer-input hidden states of the fold gate (below)
  stream [seed, 19, c]    stand-in fp32 logits for the commit (draw_logits)
  stream [seed, 20]       drafted blocks for rejection sampling (draw_trays)
All floats are drawn in fp32 and rounded to bfloat16 (round to nearest even).

Layer-input hidden states for SpecFold's parent-child gate (Sec. 3.1
Observation 1 and Fig. 6: a child's hidden state stays close to its
parent's, with the divergence at masked and newly unmasked positions):
H_0[n] ~ N(0, 1)^D; a draft's H_i[n] = H_par(i)[n] + sigma * N(0, 1)^D with
sigma = 1 where the draft unmasked n, LogU(0.02, 0.5) where n is still
masked, LogU(0.005, 0.05) where the parent already holds a token.
"""
from __future__ import annotations

import dataclasses
import hashlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MASK = -1  # the mask token [M]

_W_CHUNK = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    """One verification-step workload (sizes, tree shape and sampling setup)."""
    index: int
    name: str
    B1: int            # branches: main + B drafts
    tree: str          # "chain" | "random" | "star"
    N: int             # block length
    L: int             # shared context length
    Hq: int
    Hkv: int
    d: int
    D: int             # hidden size
    V: int             # vocabulary
    mask_frac: float   # target masked fraction (ignored when m0 is set)
    S_t: int           # max newly unmasked positions per draft
    T: float           # sampling temperature (0 = greedy)
    w_std: float
    m0: int | None = None
    # seeds of the Gumbel noise: seed = index, step0 = 100 + index, pos0 = L
    @property
    def seed(self) -> int:
        return self.index

    @property
    def step0(self) -> int:
        return 100 + self.index

    @property
    def pos0(self) -> int:
        return self.L

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload(1, "tiny_chain3_n8_l64", 3, "chain", 8, 64, 4, 2, 32, 128, 512,
                0.0, 2, 0.0, 1.0, m0=5),
    2: Workload(2, "sdar8b_budget8_n32_l256", 9, "random", 32, 256, 32, 8, 128,
                4096, 151936, 0.5, 2, 0.0, 0.02),
    3: Workload(3, "sdar8b_budget20_n32_l768_t1", 21, "random", 32, 768, 32, 8,
                128, 4096, 151936, 0.6, 2, 1.0, 0.02),
    4: Workload(4, "d3d_packed_24x16_l2048", 24, "star", 16, 2048, 32, 8, 128,
                4096, 151936, 1.0, 0, 0.0, 0.02),
    5: Workload(5, "qwen32b_wide_n64_l4096_t1", 33, "random", 64, 4096, 64, 8,
                128, 5120, 151936, 0.7, 4, 1.0, 0.02),
}


def scaled(wl: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes replaced (for small parity cases)."""
    return dataclasses.replace(wl, **kw)


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (format conversion only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16, nearest-even; returns the raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rnd) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *tag: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), *[int(t) for t in tag]])


def _normal_bf16(seed: int, tag: int, shape, std: float = 1.0) -> np.ndarray:
    x = _rng(seed, tag).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x).reshape(shape)


# ----------------------------------------------------------------------------
# tree and block states
# ----------------------------------------------------------------------------
def draw_tree(B1: int, kind: str, seed: int) -> np.ndarray:
    parent = np.full(B1, -1, dtype=np.int32)
    rng = _rng(seed, 1)
    for i in range(1, B1):
        if kind == "chain":
            parent[i] = i - 1
        elif kind == "star":
            parent[i] = 0
        elif kind == "random":
            parent[i] = rng.integers(0, i)
        else:
            raise ValueError(kind)
    return parent


def draw_states(wl: Workload, parent: np.ndarray, seed: int) -> np.ndarray:
    """Block states int32 [B1][N]; MASK = -1; drafts extend their parent."""
    B1, N, V, S_t = wl.B1, wl.N, wl.V, wl.S_t
    rs = _rng(seed, 2)
    s = np.zeros(B1, dtype=np.int64)
    for i in range(1, B1):
        s[i] = rs.integers(1, S_t + 1) if S_t >= 1 else 0
    cum = np.zeros(B1, dtype=np.int64)
    for i in range(1, B1):
        cum[i] = cum[parent[i]] + s[i]
    if wl.m0 is not None:
        m0 = wl.m0
    else:
        m0 = int(np.clip(round(wl.mask_frac * N + cum.mean()), 1, N))
    rng = _rng(seed, 3)
    state = np.empty((B1, N), dtype=np.int32)
    main = rng.integers(0, V, N).astype(np.int32)
    main[rng.choice(N, m0, replace=False)] = MASK
    state[0] = main
    for i in range(1, B1):
        row = state[parent[i]].copy()
        free = np.flatnonzero(row == MASK)
        k = int(min(s[i], free.size))
        if k:
            pick = rng.choice(free, k, replace=False)
            row[pick] = rng.integers(0, V, k).astype(np.int32)
        state[i] = row
    return state


# ----------------------------------------------------------------------------
# full input set
# ----------------------------------------------------------------------------
def draw_w(wl: Workload, seed: int | None = None, threads: int = 8) -> np.ndarray:
    """LM-head weight, bf16 bits [V][D], N(0, w_std), drawn in row chunks."""
    seed = wl.seed if seed is None else seed
    V, D = wl.V, wl.D
    out = np.empty((V, D), dtype=np.uint16)

    def one(c):
        r0 = c * _W_CHUNK
        r1 = min(V, r0 + _W_CHUNK)
        x = _rng(seed, 16, c).standard_normal((r1 - r0) * D, dtype=np.float32)
        x *= np.float32(wl.w_std)
        out[r0:r1] = f32_to_bf16_bits(x).reshape(r1 - r0, D)

    n_chunks = (V + _W_CHUNK - 1) // _W_CHUNK
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(n_chunks)))
    return out


def draw_inputs(wl: Workload, seed: int | None = None, with_w: bool = True) -> dict:
    """All inputs of one verification step as host arrays (bf16 as uint16 bits)."""
    seed = wl.seed if seed is None else seed
    parent = draw_tree(wl.B1, wl.tree, seed)
    state = draw_states(wl, parent, seed)
    B1, N, L, Hq, Hkv, d = wl.B1, wl.N, wl.L, wl.Hq, wl.Hkv, wl.d
    inp = dict(
        parent=parent,
        state=state,
        q=_normal_bf16(seed, 10, (B1, N, Hq, d)),
        k_blk=_normal_bf16(seed, 11, (B1, N, Hkv, d)),
        v_blk=_normal_bf16(seed, 12, (B1, N, Hkv, d)),
        k_ctx=_normal_bf16(seed, 13, (Hkv, L, d)),
        v_ctx=_normal_bf16(seed, 14, (Hkv, L, d)),
        hidden=_normal_bf16(seed, 15, (B1 * N, wl.D)),
    )
    if with_w:
        inp["w"] = draw_w(wl, seed)
    return inp


def draw_fold_hidden(wl: Workload, parent: np.ndarray, state: np.ndarray,
                     seed: int | None = None) -> np.ndarray:
    """bf16 bits [B1][N][D]: layer-input hidden states with the parent-child
    structure described in the module docstring."""
    seed = wl.seed if seed is None else seed
    B1, N, D = wl.B1, wl.N, wl.D
    rz = _rng(seed, 17)
    rs = _rng(seed, 18)
    H = np.empty((B1, N, D), dtype=np.float32)
    H[0] = rz.standard_normal((N, D), dtype=np.float32)
    H[0] = bf16_bits_to_f32(f32_to_bf16_bits(H[0]))
    for i in range(1, B1):
        p = int(parent[i])
        fresh = (state[p] == MASK) & (state[i] != MASK)
        masked = state[i] == MASK
        sig = np.exp(rs.uniform(np.log(0.005), np.log(0.05), N))
        sig = np.where(masked, np.exp(rs.uniform(np.log(0.02), np.log(0.5), N)), sig)
        sig = np.where(fresh, 1.0, sig).astype(np.float32)
        H[i] = H[p] + sig[:, None] * rz.standard_normal((N, D), dtype=np.float32)
        H[i] = bf16_bits_to_f32(f32_to_bf16_bits(H[i]))
    return f32_to_bf16_bits(H)


def draw_logits(M: int, V: int, seed: int, chunk: int = 64) -> np.ndarray:
    """fp32 [M][V] stand-in logits for testing the commit on its own: N(0, 1)
    rows scaled by a per-row sharpness s ~ LogU(0.5, 8), so the row
    confidences range from near-uniform to peaked."""
    out = np.empty((M, V), dtype=np.float32)
    for c0 in range(0, M, chunk):
        rng = _rng(seed, 19, c0 // chunk)
        rows = min(chunk, M - c0)
        sharp = np.exp(rng.uniform(np.log(0.5), np.log(8.0), (rows, 1))).astype(np.float32)
        out[c0:c0 + rows] = rng.standard_normal((rows, V), dtype=np.float32) * sharp
    return out


def draw_trays(n_trays: int, B: int, V: int, seed: int, T: float = 1.0, drift: float = 0.8):
    """Drafted blocks for rejection-sampling verification (stream [seed, 20]):
    target logits [n][B+1][V] (draw_logits), a proposal q [n][B][V] = the
    softmax of the target's logits at temperature T (1 when T = 0) plus
    N(0, drift^2) noise per entry (fp32, normalised), and tokens [n][B] drawn
    from q.  Returns (logits, q, tokens)."""
    rng = _rng(seed, 20)
    logits = draw_logits(n_trays * (B + 1), V, seed + 7919).reshape(n_trays, B + 1, V)
    q = np.empty((n_trays, B, V), dtype=np.float32)
    tokens = np.empty((n_trays, B), dtype=np.int32)
    t_eff = T if T > 0 else 1.0
    for j in range(n_trays):
        z = logits[j, :B].astype(np.float64) / t_eff + drift * rng.standard_normal((B, V))
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        qj = e / e.sum(axis=1, keepdims=True)
        q[j] = qj.astype(np.float32)
        g = rng.gumbel(size=(B, V))
        tokens[j] = np.argmax(np.log(np.maximum(qj, 1e-300)) + g, axis=1)
    return logits, q, tokens


def masked_count(state: np.ndarray) -> int:
    return int((state == MASK).sum())


# ----------------------------------------------------------------------------
# state-keyed stand-ins for a target model (used to plant matching drafts)
# ----------------------------------------------------------------------------
def _state_key(state_row: np.ndarray) -> int:
    h = hashlib.blake2b(np.ascontiguousarray(state_row, dtype=np.int32).tobytes(), digest_size=8)
    return int.from_bytes(h.digest(), "little")


def state_keyed_logits(seed: int, state_row: np.ndarray, V: int, scale: float = 1.28) -> np.ndarray:
    """fp32 logits [N][V] that depend only on the block state (a toy target).

    Two branches holding the same state receive the same logits, as a real
    target would give them; different states receive unrelated draws."""
    N = state_row.shape[0]
    rng = _rng(seed, 40, _state_key(state_row) & 0x7FFFFFFFFFFFFFFF)
    x = rng.standard_normal((N, V), dtype=np.float32)
    x *= np.float32(scale)
    return x


def state_keyed_hidden(seed: int, state: np.ndarray, D: int) -> np.ndarray:
    """bf16 bits [B1*N][D] hidden rows that depend only on each branch's state."""
    B1, N = state.shape
    out = np.empty((B1 * N, D), dtype=np.uint16)
    for i in range(B1):
        rng = _rng(seed, 41, _state_key(state[i]) & 0x7FFFFFFFFFFFFFFF)
        out[i * N:(i + 1) * N] = f32_to_bf16_bits(rng.standard_normal((N, D), dtype=np.float32))
    return out
