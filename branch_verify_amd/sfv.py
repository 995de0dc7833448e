"""ctypes binding of libsfv (include/sfv.h): the same names, argument
marshalling only.  Tensors are torch device tensors; every computation runs
in the library's HIP kernels.  Loading fails loudly when the library has not
been built."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsfv.so")

SFV_OK = 0
SFV_E_INVAL = -1
SFV_E_UNSUPPORTED = -2
SFV_E_TREE = -3
SFV_E_STATE = -4
SFV_E_WORKSPACE = -5
SFV_E_HIP = -6
SFV_MASK = -1

EXPORTS = [
    "sfv_last_error", "sfv_version", "sfv_attend_workspace_bytes", "sfv_attend_branches",
    "sfv_masked_rows", "sfv_lm_head", "sfv_commit_workspace_bytes", "sfv_commit",
    "sfv_match_tree", "sfv_selfcheck_bounds", "sfv_fold_gate", "sfv_attend_folded_workspace_bytes",
    "sfv_attend_folded", "sfv_stale_topk_workspace_bytes", "sfv_stale_topk", "sfv_draft_tree",
    "sfv_attend_trays", "sfv_reject_workspace_bytes", "sfv_reject_verify", "sfv_match_trays",
    "sfv_lm_head_greedy_bytes", "sfv_lm_head_greedy", "sfv_commit_greedy_workspace_bytes",
    "sfv_commit_greedy", "sfv_commit_noalloc", "sfv_gumbel_words",
]

_lib = None


class SfvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libsfv error {code}: {msg}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load libsfv.so (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    try:
        import torch  # noqa: F401  (its HIP runtime must be the one libsfv binds to)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    SZ = ctypes.c_size_t
    F = ctypes.c_float
    U64 = ctypes.c_uint64
    I64 = ctypes.c_int64
    lib.sfv_last_error.restype = ctypes.c_char_p
    lib.sfv_last_error.argtypes = []
    lib.sfv_version.restype = I
    lib.sfv_attend_workspace_bytes.argtypes = [I, I, I, I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_attend_branches.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, SZ, P]
    lib.sfv_masked_rows.argtypes = [P, I, I, P, P, P]
    lib.sfv_reject_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_reject_verify.argtypes = [P, P, P, I, I, I, F, U64, U64, I64, P, P, P, SZ, P]
    lib.sfv_match_trays.argtypes = [P, P, I, P, P, I, P, P]
    lib.sfv_attend_trays.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, SZ, P]
    lib.sfv_lm_head.argtypes = [P, P, I, I, P, I, I, P, P, P]
    lib.sfv_commit_workspace_bytes.argtypes = [I, I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_commit.argtypes = [P, P, I, P, P, I, I, I, F, U64, U64, I64, I, F, P, P, P, P, P, SZ, P]
    lib.sfv_commit_noalloc.argtypes = [P, P, I, P, P, I, I, I, F, U64, U64, I64, I, F, P, P, P, P, P]
    lib.sfv_match_tree.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P]
    lib.sfv_lm_head_greedy_bytes.argtypes = [I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_lm_head_greedy.argtypes = [P, P, I, I, P, I, I, P, P, SZ, P, P]
    lib.sfv_commit_greedy_workspace_bytes.argtypes = [I, I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_commit_greedy.argtypes = [P, SZ, I, P, P, I, P, P, I, I, I, I, F, P, P, P, P, P, SZ, P]
    lib.sfv_selfcheck_bounds.argtypes = [P, P]
    lib.sfv_gumbel_words.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P, P]
    lib.sfv_stale_topk_workspace_bytes.argtypes = [I, I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_stale_topk.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, SZ, P]
    lib.sfv_draft_tree.argtypes = [P, P, P, P, I, I, I, I, F, U64, U64, I64, P, P, P, P]
    lib.sfv_fold_gate.argtypes = [P, P, I, I, I, F, P, P, P, P, P, P, P]
    lib.sfv_attend_folded_workspace_bytes.argtypes = [I, I, I, I, I, I, ctypes.POINTER(SZ)]
    lib.sfv_attend_folded.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, P, P, P, P, SZ, P]
    for name in EXPORTS:
        if name not in ("sfv_last_error", "sfv_version"):
            getattr(lib, name).restype = I
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int):
    if rc != SFV_OK:
        raise SfvError(rc, _lib.sfv_last_error().decode())
    return rc


def last_error() -> str:
    return load().sfv_last_error().decode()


def sfv_version() -> int:
    return load().sfv_version()


def sfv_attend_workspace_bytes(B1, N, L, Hq, Hkv, d) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_attend_workspace_bytes(B1, N, L, Hq, Hkv, d, ctypes.byref(out)))
    return out.value


def sfv_attend_branches(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d, softmax_scale,
                        o, lse, workspace=None, workspace_bytes=0, stream=None):
    return _check(load().sfv_attend_branches(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx), B1, N, L, Hq, Hkv, d,
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def sfv_attend_trays(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d, softmax_scale, o, lse,
                     workspace=None, workspace_bytes=0, stream=None):
    return _check(load().sfv_attend_trays(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx), B1, N, L, Hq, Hkv, d,
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def sfv_masked_rows(state, B1, N, rows, count, stream=None):
    return _check(load().sfv_masked_rows(_ptr(state), B1, N, _ptr(rows), _ptr(count), _stream(stream)))


def sfv_lm_head(hidden, rows, M, R, w, D, V, logits, stream=None, status=None):
    return _check(load().sfv_lm_head(_ptr(hidden), _ptr(rows), M, R, _ptr(w), D, V, _ptr(logits),
                                     _ptr(status), _stream(stream)))


def sfv_commit_workspace_bytes(B1, N, M, V) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_commit_workspace_bytes(B1, N, M, V, ctypes.byref(out)))
    return out.value


def _host_i32(seq):
    arr = (ctypes.c_int32 * len(seq))(*[int(x) for x in seq])
    return arr


def sfv_commit(logits, rows, M, state, parent_host, B1, N, V, temperature, seed, step0, pos0,
               k_max, tau, next_state, commit_pos, token, conf, workspace, workspace_bytes,
               stream=None):
    par = _host_i32(parent_host)
    return _check(load().sfv_commit(
        _ptr(logits), _ptr(rows), M, _ptr(state), ctypes.cast(par, ctypes.c_void_p), B1, N, V,
        float(temperature), int(seed) & (2**64 - 1), int(step0) & (2**64 - 1), int(pos0), k_max,
        float(tau), _ptr(next_state), _ptr(commit_pos), _ptr(token), _ptr(conf), _ptr(workspace),
        int(workspace_bytes), _stream(stream)))


def sfv_commit_noalloc(logits, rows, M, state, parent_host, B1, N, V, temperature, seed, step0, pos0,
                       k_max, tau, next_state, commit_pos, token, conf, stream=None):
    par = _host_i32(parent_host)
    return _check(load().sfv_commit_noalloc(
        _ptr(logits), _ptr(rows), M, _ptr(state), ctypes.cast(par, ctypes.c_void_p), B1, N, V,
        float(temperature), int(seed) & (2**64 - 1), int(step0) & (2**64 - 1), int(pos0), k_max,
        float(tau), _ptr(next_state), _ptr(commit_pos), _ptr(token), _ptr(conf), _stream(stream)))


def sfv_lm_head_greedy_bytes(M, V, D) -> int:
    """Bytes of the strip partials, or 0 where the shape is not served."""
    lib = load()
    out = ctypes.c_size_t(0)
    rc = lib.sfv_lm_head_greedy_bytes(M, V, D, ctypes.byref(out))
    if rc == SFV_E_UNSUPPORTED:
        return 0
    _check(rc)
    return out.value


def sfv_lm_head_greedy(hidden, rows, M, R, w, D, V, logits, partials, partials_bytes, stream=None,
                       status=None):
    return _check(load().sfv_lm_head_greedy(_ptr(hidden), _ptr(rows), M, R, _ptr(w), D, V, _ptr(logits),
                                            _ptr(partials), int(partials_bytes), _ptr(status), _stream(stream)))


def sfv_commit_greedy_workspace_bytes(B1, N, M, V) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_commit_greedy_workspace_bytes(B1, N, M, V, ctypes.byref(out)))
    return out.value


def sfv_commit_greedy(partials, partials_bytes, D, logits, rows, M, state, parent_host, B1, N, V, k_max, tau,
                      next_state, commit_pos, token, conf, workspace, workspace_bytes, stream=None):
    par = _host_i32(parent_host)
    return _check(load().sfv_commit_greedy(
        _ptr(partials), int(partials_bytes), D, _ptr(logits), _ptr(rows), M, _ptr(state),
        ctypes.cast(par, ctypes.c_void_p), B1, N, V, k_max, float(tau), _ptr(next_state), _ptr(commit_pos),
        _ptr(token), _ptr(conf), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sfv_match_tree(state, next_state, commit_pos, parent_host, B1, N, k_max, S_max, chain,
                   n_accepted, status, stream=None):
    par = _host_i32(parent_host)
    return _check(load().sfv_match_tree(
        _ptr(state), _ptr(next_state), _ptr(commit_pos), ctypes.cast(par, ctypes.c_void_p), B1, N,
        k_max, S_max, _ptr(chain), _ptr(n_accepted), _ptr(status), _stream(stream)))


def sfv_gumbel_words(first, count, out, stream=None):
    return _check(load().sfv_gumbel_words(int(first), int(count), _ptr(out), _stream(stream)))


def sfv_selfcheck_bounds(out, stream=None):
    return _check(load().sfv_selfcheck_bounds(_ptr(out), _stream(stream)))


def sfv_fold_gate(hidden, parent_host, B1, N, D, delta, recompute, src, rec_rows, rec_count,
                  rec_pos, branch_off, stream=None):
    par = _host_i32(parent_host)
    return _check(load().sfv_fold_gate(
        _ptr(hidden), ctypes.cast(par, ctypes.c_void_p), B1, N, D, float(delta), _ptr(recompute),
        _ptr(src), _ptr(rec_rows), _ptr(rec_count), _ptr(rec_pos), _ptr(branch_off), _stream(stream)))


def sfv_attend_folded_workspace_bytes(B1, N, L, Hq, Hkv, d) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_attend_folded_workspace_bytes(B1, N, L, Hq, Hkv, d, ctypes.byref(out)))
    return out.value


def sfv_attend_folded(q, k_blk, v_blk, k_ctx, v_ctx, B1, N, L, Hq, Hkv, d, softmax_scale, src,
                      rec_rows, rec_count, rec_pos, o, lse, workspace=None, workspace_bytes=0,
                      stream=None):
    return _check(load().sfv_attend_folded(
        _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ctx), _ptr(v_ctx), B1, N, L, Hq, Hkv, d,
        float(softmax_scale), _ptr(src), _ptr(rec_rows), _ptr(rec_count), _ptr(rec_pos), _ptr(o),
        _ptr(lse), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sfv_stale_topk_workspace_bytes(M, V, N, K) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_stale_topk_workspace_bytes(M, V, N, K, ctypes.byref(out)))
    return out.value


def sfv_stale_topk(logits, rows, conf, M, V, N, branch, K, top_ids, top_logit, conf_pos, workspace,
                   workspace_bytes, stream=None):
    return _check(load().sfv_stale_topk(
        _ptr(logits), _ptr(rows), _ptr(conf), M, V, N, branch, K, _ptr(top_ids), _ptr(top_logit),
        _ptr(conf_pos), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sfv_draft_tree(root, top_ids, top_logit, conf, N, K, D, W, temperature, seed, step0, pos0,
                   parent, states, n_drafts, stream=None):
    return _check(load().sfv_draft_tree(
        _ptr(root), _ptr(top_ids), _ptr(top_logit), _ptr(conf), N, K, D, W, float(temperature),
        int(seed) & (2**64 - 1), int(step0) & (2**64 - 1), int(pos0), _ptr(parent), _ptr(states),
        _ptr(n_drafts), _stream(stream)))


def sfv_reject_workspace_bytes(n_trays, B, V) -> int:
    out = ctypes.c_size_t(0)
    _check(load().sfv_reject_workspace_bytes(n_trays, B, V, ctypes.byref(out)))
    return out.value


def sfv_reject_verify(logits, q, tokens, n_trays, B, V, temperature, seed, step0, pos0, n_accept,
                      next_token, workspace, workspace_bytes, stream=None):
    return _check(load().sfv_reject_verify(
        _ptr(logits), _ptr(q), _ptr(tokens), n_trays, B, V, float(temperature),
        int(seed) & (2**64 - 1), int(step0) & (2**64 - 1), int(pos0), _ptr(n_accept),
        _ptr(next_token), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def sfv_match_trays(n_accept, next_token, verified, tray_k, tray_alt, n_prepared, served, stream=None):
    return _check(load().sfv_match_trays(
        _ptr(n_accept), _ptr(next_token), verified, _ptr(tray_k), _ptr(tray_alt), n_prepared,
        _ptr(served), _stream(stream)))
