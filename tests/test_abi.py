"""The C ABI on the host: the library loads without a GPU, exports every
entry point include/sfv.h declares, and rejects bad arguments synchronously
(each check runs before anything is enqueued, so no GPU is touched)."""
import ctypes
import os
import re

import pytest

from branch_verify_amd import sfv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sfv.LIB_PATH):
        pytest.fail("libsfv.so is not built (run __graft_entry__.build())")
    return sfv.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(sfv.EXPORTS)


def test_version_and_empty_error(lib):
    assert lib.sfv_version() >= 100


def _ws(fn, *args):
    out = ctypes.c_size_t(0)
    return fn(*args, ctypes.byref(out)), out.value


def test_attend_workspace_validation(lib):
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 8, 64, 4, 2, 32)[0] == sfv.SFV_OK
    assert _ws(lib.sfv_attend_workspace_bytes, 0, 8, 64, 4, 2, 32)[0] == sfv.SFV_E_INVAL
    assert _ws(lib.sfv_attend_workspace_bytes, 65, 8, 64, 4, 2, 32)[0] == sfv.SFV_E_INVAL
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 257, 64, 4, 2, 32)[0] == sfv.SFV_E_INVAL
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 8, -1, 4, 2, 32)[0] == sfv.SFV_E_INVAL
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 8, 64, 6, 4, 32)[0] == sfv.SFV_E_INVAL
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 8, 64, 48, 3, 32)[0] == sfv.SFV_E_UNSUPPORTED
    assert _ws(lib.sfv_attend_workspace_bytes, 3, 8, 64, 4, 2, 96)[0] == sfv.SFV_E_UNSUPPORTED
    assert b"96" in lib.sfv_last_error()
    assert lib.sfv_attend_workspace_bytes(3, 8, 64, 4, 2, 32, None) == sfv.SFV_E_INVAL


@pytest.mark.parametrize("B1,N,L,Hq,Hkv,d,splits", [
    (9, 32, 256, 32, 8, 128, 1),      # SDAR-8B-like budget 8: one split, no partial state
    (21, 32, 768, 32, 8, 128, 1),     # budget 20
    (24, 16, 2048, 32, 8, 128, 4),    # D3D-style packed trays: 96 row tiles x heads, 512 keys a split
    (33, 64, 4096, 64, 8, 128, 1),    # Qwen3-32B-like: 1056 workgroups without splitting
    (2, 5, 1500, 8, 2, 64, 2),        # 750 keys rounded up to 768 a split: 2, the last ragged
    (3, 9, 3000, 4, 4, 32, 5),        # 640 keys a split: 5
    (1, 1, 511, 1, 1, 32, 1),         # below 512 keys: never split
    (64, 64, 300, 32, 8, 64, 1),      # exactly two rounds of 512: no tail
])
def test_attend_split_plan(lib, B1, N, L, Hq, Hkv, d, splits):
    """The split planner, seen through the workspace size: at least 512 context
    keys per split, as many splits as bring the grid to 512 workgroups; one
    split needs no workspace unless the unsplit grid overshoots whole rounds
    of 512 workgroups by at most 128: then the last ceil(overshoot / Hkv) row
    tiles of every kv head are split over the context (at least two 64-key
    tiles a split, at most 8 splits, up to 512 workgroups) and only their
    states need room."""
    rc, nb = _ws(lib.sfv_attend_workspace_bytes, B1, N, L, Hq, Hkv, d)
    assert rc == sfv.SFV_OK
    rows = B1 * N * (Hq // Hkv)
    if splits > 1:
        assert nb == splits * Hkv * rows * (d + 2) * 4
        return
    wgs = -(-rows // 128) * Hkv
    over = wgs % 512
    if wgs > 512 and 0 < over <= 128 and L >= 128:
        tail = -(-over // Hkv)
        ts = min(512 // (tail * Hkv), L // 128, 8)
        chunk = -(-(-(-L // ts)) // 64) * 64
        ts = -(-L // chunk)
        assert nb == ts * Hkv * tail * 128 * (d + 2) * 4, (nb, tail, ts)
        if (B1, N, L) == (33, 64, 4096):
            assert (tail, ts) == (4, 8)
    else:
        assert nb == 0


def test_attend_rejects_before_launch(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    args = [fake] * 5 + [3, 8, 64, 4, 2, 32, ctypes.c_float(0.17), fake, fake]
    # null q
    assert lib.sfv_attend_branches(None, *args[1:], None, 0, None) == sfv.SFV_E_INVAL
    # misaligned output
    bad = list(args); bad[12] = P(0x1002)   # o
    rc, need = _ws(lib.sfv_attend_workspace_bytes, 3, 8, 64, 4, 2, 32)
    assert lib.sfv_attend_branches(*bad, fake, need, None) == sfv.SFV_E_INVAL
    # workspace too small when splits are needed
    rc, need = _ws(lib.sfv_attend_workspace_bytes, 9, 32, 4096, 32, 8, 128)
    assert need > 0
    args2 = [fake] * 5 + [9, 32, 4096, 32, 8, 128, ctypes.c_float(0.088), fake, fake]
    assert lib.sfv_attend_branches(*args2, fake, need - 1, None) == sfv.SFV_E_WORKSPACE
    # non-finite, zero or negative scale (the running max is of unscaled scores)
    for bad_scale in (float("inf"), 0.0, -0.17, -0.0):
        args3 = list(args); args3[11] = ctypes.c_float(bad_scale)
        assert lib.sfv_attend_branches(*args3, fake, 1 << 30, None) == sfv.SFV_E_INVAL
        assert lib.sfv_attend_trays(*args3, fake, 1 << 30, None) == sfv.SFV_E_INVAL


def test_lm_head_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    assert lib.sfv_lm_head(f, f, -1, 8, f, 128, 512, f, None, None) == sfv.SFV_E_INVAL
    assert lib.sfv_lm_head(f, f, 4, 8, f, 100, 512, f, None, None) == sfv.SFV_E_UNSUPPORTED
    assert lib.sfv_lm_head(None, f, 4, 8, f, 128, 512, f, None, None) == sfv.SFV_E_INVAL
    assert lib.sfv_lm_head(f, f, 4, 0, f, 128, 512, f, None, None) == sfv.SFV_E_INVAL
    assert lib.sfv_lm_head(P(0x1004), f, 4, 8, f, 128, 512, f, None, None)
    assert lib.sfv_lm_head(f, f, 4, 8, f, 128, 512, f, P(0x1002), None) == sfv.SFV_E_INVAL  # misaligned status == sfv.SFV_E_INVAL


def _commit(lib, parent, B1=3, N=8, M=4, V=512, T=0.0, k_max=1, ws_bytes=None, logits=0x1000,
            tau=0.0):
    P = ctypes.c_void_p
    f = P(0x1000)
    par = (ctypes.c_int32 * len(parent))(*parent)
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return lib.sfv_commit(P(logits), f, M, f, ctypes.cast(par, P), B1, N, V, ctypes.c_float(T),
                          ctypes.c_uint64(1), ctypes.c_uint64(2), ctypes.c_int64(3), k_max,
                          ctypes.c_float(tau), f, f, f, f, f, ws_bytes, None)


def test_commit_validation(lib):
    assert _commit(lib, [0, 0, 1]) == sfv.SFV_E_TREE
    assert _commit(lib, [-1, 1, 0]) == sfv.SFV_E_TREE
    assert _commit(lib, [-1, 0, 3]) == sfv.SFV_E_TREE
    assert _commit(lib, [-1, 0, 1], M=25) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], V=500) == sfv.SFV_E_UNSUPPORTED
    assert _commit(lib, [-1, 0, 1], T=-1.0) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], T=float("nan")) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], k_max=0) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], k_max=9) == sfv.SFV_E_INVAL  # more than N positions
    assert _commit(lib, [-1, 0, 1], k_max=2, tau=float("nan")) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], k_max=2, tau=float("inf")) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1, 0, 1], ws_bytes=16) == sfv.SFV_E_WORKSPACE
    assert _commit(lib, [-1, 0, 1], logits=0x1004) == sfv.SFV_E_INVAL
    assert _commit(lib, [-1] + [0] * 64, B1=65) == sfv.SFV_E_INVAL


def test_greedy_partials_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    # from 33 rows on: one 16-byte partial per row and 256-id vocab tile
    rc, nb = _ws(lib.sfv_lm_head_greedy_bytes, 148, 151936, 4096)
    assert rc == sfv.SFV_OK and nb == (151936 + 255) // 256 * 148 * 16
    rc, nb = _ws(lib.sfv_lm_head_greedy_bytes, 193, 151936, 4096)
    assert rc == sfv.SFV_OK and nb == (151936 + 255) // 256 * 193 * 16
    rc, nb = _ws(lib.sfv_lm_head_greedy_bytes, 160, 1000, 128)
    assert rc == sfv.SFV_OK and nb == 4 * 160 * 16
    rc, nb = _ws(lib.sfv_lm_head_greedy_bytes, 161, 1000, 64)
    assert rc == sfv.SFV_OK and nb == 4 * 161 * 16
    for M, D in [(32, 128), (0, 128), (148, 100), (257, 100), (1, 64)]:
        assert _ws(lib.sfv_lm_head_greedy_bytes, M, 512, D)[0] == sfv.SFV_E_UNSUPPORTED, (M, D)
    for M in (33, 64, 148, 257):  # D = 64 at every supported row count
        rc, nb = _ws(lib.sfv_lm_head_greedy_bytes, M, 1000, 64)
        assert rc == sfv.SFV_OK and nb == 4 * M * 16, M
    assert _ws(lib.sfv_lm_head_greedy_bytes, -1, 512, 128)[0] == sfv.SFV_E_INVAL
    assert lib.sfv_lm_head_greedy_bytes(148, 512, 128, None) == sfv.SFV_E_INVAL
    nb = _ws(lib.sfv_lm_head_greedy_bytes, 148, 512, 128)[1]
    g = lib.sfv_lm_head_greedy
    assert g(f, f, 32, 200, f, 128, 512, f, f, nb, None, None) == sfv.SFV_E_UNSUPPORTED
    assert g(None, f, 148, 200, f, 128, 512, f, f, nb, None, None) == sfv.SFV_E_INVAL
    assert g(f, f, 148, 200, f, 128, 512, f, None, nb, None, None) == sfv.SFV_E_INVAL
    assert g(f, f, 148, 0, f, 128, 512, f, f, nb, None, None) == sfv.SFV_E_INVAL
    assert g(f, f, 148, 200, f, 128, 512, f, P(0x1008), nb, None, None) == sfv.SFV_E_INVAL
    assert g(f, f, 148, 200, f, 128, 512, f, f, nb - 16, None, None) == sfv.SFV_E_WORKSPACE
    assert g(f, f, 148, 200, f, 128, 512, f, f, nb, P(0x1001), None) == sfv.SFV_E_INVAL  # misaligned status


def test_step_attention_placement():
    """The automatic attention placement of the workload shapes."""
    import types

    from branch_verify_amd.step import VerifyStep
    place = VerifyStep.attn_placement

    def shape(B1, N, L, Hq, d=128):
        return types.SimpleNamespace(B1=B1, N=N, L=L, Hq=Hq, d=d, M=0)
    # the SDAR-8B-like, D3D-style and Qwen3-32B-like steps: only the last one's
    # attention (about 0.29 TFLOP) is long enough to overlap
    assert place(shape(9, 32, 256, 32)) == "in_order"
    assert place(shape(21, 32, 768, 32)) == "in_order"
    assert place(shape(24, 16, 2048, 32)) == "in_order"
    assert place(shape(33, 64, 4096, 64)) == "commit"
    assert place(shape(9, 32, 256, 32), "lm_head") == "lm_head"
    with pytest.raises(ValueError):
        place(shape(9, 32, 256, 32), "beside")


def _commit_greedy(lib, parent, B1=9, N=32, M=148, V=512, D=128, k_max=1, tau=0.0, ws_bytes=None,
                   parts_bytes=None, logits=0x1000):
    P = ctypes.c_void_p
    f = P(0x1000)
    par = (ctypes.c_int32 * len(parent))(*parent)
    if parts_bytes is None:
        parts_bytes = 1 << 30
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return lib.sfv_commit_greedy(f, parts_bytes, D, P(logits), f, M, f, ctypes.cast(par, P), B1, N, V, k_max,
                                 ctypes.c_float(tau), f, f, f, f, f, ws_bytes, None)


def test_commit_greedy_validation(lib):
    par = [-1] + list(range(8))
    assert _ws(lib.sfv_commit_greedy_workspace_bytes, 9, 32, 148, 512)[0] == sfv.SFV_OK
    assert _ws(lib.sfv_commit_greedy_workspace_bytes, 9, 32, 300, 512)[0] == sfv.SFV_E_INVAL
    need = _ws(lib.sfv_commit_greedy_workspace_bytes, 9, 32, 148, 512)[1]
    assert _commit_greedy(lib, [0] * 9) == sfv.SFV_E_TREE
    assert _commit_greedy(lib, par, M=32) == sfv.SFV_E_UNSUPPORTED    # the tiled kernel writes no partials
    assert _commit_greedy(lib, par, V=500) == sfv.SFV_E_UNSUPPORTED
    assert _commit_greedy(lib, par, D=100) == sfv.SFV_E_UNSUPPORTED
    assert _commit_greedy(lib, par, k_max=0) == sfv.SFV_E_INVAL
    assert _commit_greedy(lib, par, k_max=33) == sfv.SFV_E_INVAL
    assert _commit_greedy(lib, par, k_max=2, tau=float("nan")) == sfv.SFV_E_INVAL
    assert _commit_greedy(lib, par, ws_bytes=need - 1) == sfv.SFV_E_WORKSPACE
    assert _commit_greedy(lib, par, parts_bytes=16) == sfv.SFV_E_WORKSPACE
    assert _commit_greedy(lib, par, logits=0x1004) == sfv.SFV_E_INVAL


def test_commit_workspace_covers_every_tree(lib):
    for (B1, N, M, V) in [(3, 8, 10, 512), (9, 32, 144, 151936), (33, 64, 1478, 151936), (64, 256, 16384, 8)]:
        rc, need = _ws(lib.sfv_commit_workspace_bytes, B1, N, M, V)
        assert rc == sfv.SFV_OK and need > 0
    assert _ws(lib.sfv_commit_workspace_bytes, 3, 8, 30, 512)[0] == sfv.SFV_E_INVAL


def test_match_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    par = (ctypes.c_int32 * 3)(-1, 0, 2)
    assert lib.sfv_match_tree(f, f, f, ctypes.cast(par, P), 3, 8, 1, 2, f, f, f, None) == sfv.SFV_E_TREE
    par = (ctypes.c_int32 * 3)(-1, 0, 1)
    assert lib.sfv_match_tree(f, f, f, ctypes.cast(par, P), 3, 0, 1, 2, f, f, f, None) == sfv.SFV_E_INVAL
    assert lib.sfv_match_tree(None, f, f, ctypes.cast(par, P), 3, 8, 1, 2, f, f, f, None) == sfv.SFV_E_INVAL
    assert lib.sfv_match_tree(f, f, f, None, 3, 8, 1, 2, f, f, f, None) == sfv.SFV_E_INVAL


def test_masked_rows_validation(lib):
    f = ctypes.c_void_p(0x1000)
    assert lib.sfv_masked_rows(None, 3, 8, f, f, None) == sfv.SFV_E_INVAL
    assert lib.sfv_masked_rows(f, 0, 8, f, f, None) == sfv.SFV_E_INVAL
    assert lib.sfv_masked_rows(f, 3, 300, f, f, None) == sfv.SFV_E_INVAL


def test_single_hip_runtime_in_process(lib):
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) <= 1, libs


def test_fold_gate_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    par = (ctypes.c_int32 * 3)(-1, 0, 1)
    pp = ctypes.cast(par, P)
    F = ctypes.c_float

    def call(h=f, tree=pp, N=8, D=64, delta=0.1, last=f):
        return lib.sfv_fold_gate(h, tree, 3, N, D, F(delta), f, f, f, f, f, last, None)

    assert call(last=None) == sfv.SFV_E_INVAL
    assert call(D=60) == sfv.SFV_E_UNSUPPORTED
    assert call(delta=float("nan")) == sfv.SFV_E_INVAL
    assert call(h=P(0x1008)) == sfv.SFV_E_INVAL
    assert call(N=0) == sfv.SFV_E_INVAL
    bad = (ctypes.c_int32 * 3)(-1, 2, 0)
    assert call(tree=ctypes.cast(bad, P)) == sfv.SFV_E_TREE


def test_attend_folded_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    F = ctypes.c_float

    def call(q=f, B1=3, G=(4, 2), d=32, scale=0.17, src=f, ws=1 << 30, o=f, N=8, rec_pos=f):
        return lib.sfv_attend_folded(q, f, f, f, f, B1, N, 64, G[0], G[1], d, F(scale), src, f, f,
                                     rec_pos, o, f, f, ws, None)

    assert call(q=None) == sfv.SFV_E_INVAL
    assert call(src=None) == sfv.SFV_E_INVAL
    assert call(rec_pos=None) == sfv.SFV_E_INVAL
    assert call(d=96) == sfv.SFV_E_UNSUPPORTED
    assert call(G=(48, 3)) == sfv.SFV_E_UNSUPPORTED
    assert call(scale=float("nan")) == sfv.SFV_E_INVAL
    assert call(scale=0.0) == sfv.SFV_E_INVAL
    assert call(scale=-0.17) == sfv.SFV_E_INVAL
    assert call(o=P(0x1002)) == sfv.SFV_E_INVAL
    assert call(B1=0) == sfv.SFV_E_INVAL
    assert call(N=257) == sfv.SFV_E_INVAL
    rc, need = _ws(lib.sfv_attend_folded_workspace_bytes, 3, 8, 64, 4, 2, 32)
    assert rc == sfv.SFV_OK and need > 0          # context states even with one split
    assert call(ws=need - 1) == sfv.SFV_E_WORKSPACE
    rc, need0 = _ws(lib.sfv_attend_folded_workspace_bytes, 3, 8, 0, 4, 2, 32)
    assert rc == sfv.SFV_OK and need0 == 0        # no context, no workspace
    assert _ws(lib.sfv_attend_folded_workspace_bytes, 3, 8, 64, 4, 2, 96)[0] == sfv.SFV_E_UNSUPPORTED


def test_stale_topk_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)

    def call(M=4, V=512, N=8, branch=0, K=32, ptr=f, ws=1 << 30, wsp=f):
        return lib.sfv_stale_topk(ptr, f, f, M, V, N, branch, K, f, f, f, wsp, ws, None)

    assert call(K=0) == sfv.SFV_E_INVAL
    assert call(K=33) == sfv.SFV_E_INVAL
    assert call(V=16, K=32) == sfv.SFV_E_INVAL
    assert call(N=0) == sfv.SFV_E_INVAL
    assert call(branch=-1) == sfv.SFV_E_INVAL
    assert call(M=-1) == sfv.SFV_E_INVAL
    assert call(ptr=None) == sfv.SFV_E_INVAL
    assert call(wsp=P(0x1008)) == sfv.SFV_E_INVAL
    rc, need = _ws(lib.sfv_stale_topk_workspace_bytes, 4, 151936, 8, 32)
    assert rc == sfv.SFV_OK and need == 4 * 16 * 32 * 8
    assert call(V=151936, ws=need - 1) == sfv.SFV_E_WORKSPACE
    assert _ws(lib.sfv_stale_topk_workspace_bytes, 4, 16, 8, 32)[0] == sfv.SFV_E_INVAL


def test_draft_tree_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    F = ctypes.c_float

    def call(N=8, K=8, D=5, W=2, T=0.0, ptr=f):
        return lib.sfv_draft_tree(ptr, f, f, f, N, K, D, W, F(T), ctypes.c_uint64(1), ctypes.c_uint64(2),
                                  ctypes.c_int64(3), f, f, f, None)

    assert call(D=64) == sfv.SFV_E_INVAL
    assert call(D=-1) == sfv.SFV_E_INVAL
    assert call(W=17) == sfv.SFV_E_INVAL
    assert call(K=33) == sfv.SFV_E_INVAL
    assert call(N=257) == sfv.SFV_E_INVAL
    assert call(T=-1.0) == sfv.SFV_E_INVAL
    assert call(T=float("inf")) == sfv.SFV_E_INVAL
    assert call(ptr=None) == sfv.SFV_E_INVAL


def test_reject_validation(lib):
    P = ctypes.c_void_p
    f = P(0x1000)
    F = ctypes.c_float

    def call(n=4, B=16, V=512, T=1.0, ptr=f, ws=1 << 30, wsp=P(0x10000)):
        return lib.sfv_reject_verify(ptr, f, f, n, B, V, F(T), ctypes.c_uint64(1), ctypes.c_uint64(2),
                                     ctypes.c_int64(3), f, f, wsp, ws, None)

    assert call(n=0) == sfv.SFV_E_INVAL
    assert call(n=65) == sfv.SFV_E_INVAL
    assert call(B=0) == sfv.SFV_E_INVAL
    assert call(B=257) == sfv.SFV_E_INVAL
    assert call(T=-0.5) == sfv.SFV_E_INVAL
    assert call(T=float("nan")) == sfv.SFV_E_INVAL
    assert call(ptr=None) == sfv.SFV_E_INVAL
    assert call(wsp=P(0x10010)) == sfv.SFV_E_INVAL
    rc, need = _ws(lib.sfv_reject_workspace_bytes, 4, 16, 151936)
    assert rc == sfv.SFV_OK and need > 0
    assert call(V=151936, ws=need - 1) == sfv.SFV_E_WORKSPACE
    assert lib.sfv_match_trays(f, f, -1, f, f, 3, f, None) == sfv.SFV_E_INVAL
    assert lib.sfv_match_trays(f, f, 0, None, f, 3, f, None) == sfv.SFV_E_INVAL


def test_attend_trays_validation(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    args = [fake] * 5 + [3, 8, 64, 4, 2, 32, ctypes.c_float(0.17), fake, fake]
    assert lib.sfv_attend_trays(None, *args[1:], None, 0, None) == sfv.SFV_E_INVAL
    bad = list(args); bad[10] = 96
    assert lib.sfv_attend_trays(*bad, None, 0, None) == sfv.SFV_E_UNSUPPORTED


def test_commit_noalloc_limits(lib):
    """The static-workspace commit checks its arguments as sfv_commit does and
    rejects, before any device call, a shape whose workspace exceeds the
    static array (64 x 256 positions all masked at T = 0 need 1048832 bytes)."""
    P = ctypes.c_void_p
    f = P(0x1000)

    def call(parent, B1=3, N=8, M=4, V=512, T=0.0, k_max=1):
        par = (ctypes.c_int32 * len(parent))(*parent)
        return lib.sfv_commit_noalloc(f, f, M, f, ctypes.cast(par, P), B1, N, V, ctypes.c_float(T),
                                      ctypes.c_uint64(1), ctypes.c_uint64(2), ctypes.c_int64(3), k_max,
                                      ctypes.c_float(0.0), f, f, f, f, None)

    assert call([0, 0, 1]) == sfv.SFV_E_TREE
    assert call([-1, 0, 1], V=500) == sfv.SFV_E_UNSUPPORTED
    assert call([-1, 0, 1], k_max=0) == sfv.SFV_E_INVAL
    big = [-1] + [0] * 63
    assert call(big, B1=64, N=256, M=64 * 256, V=151936) == sfv.SFV_E_WORKSPACE
    assert b"static" in lib.sfv_last_error()


def test_gumbel_words_validation(lib):
    """The word range may not run past 2^32; out must be non-null and aligned."""
    P = ctypes.c_void_p
    U = ctypes.c_uint32
    assert lib.sfv_gumbel_words(U(2**32 - 4), U(5), P(0x1000), None) == sfv.SFV_E_INVAL
    assert lib.sfv_gumbel_words(U(0), U(8), None, None) == sfv.SFV_E_INVAL
    assert lib.sfv_gumbel_words(U(0), U(8), P(0x1002), None) == sfv.SFV_E_INVAL
