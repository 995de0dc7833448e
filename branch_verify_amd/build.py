"""Builds libsfv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every HIP source is compiled with hipcc --offload-arch=gfx950; the commit
kernels are compiled without floating-point contraction so that their exact
decisions round as defined.  The library is linked against the HIP runtime
that PyTorch ships (RPATH to torch/lib), so one runtime serves both.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsfv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = {
    "api.cpp": [],
    "attention.hip": [],
    "lm_head.hip": [],
    "commit.hip": ["-ffp-contract=off"],
    "match.hip": [],
    "fold.hip": ["-ffp-contract=off"],
    "draft.hip": ["-ffp-contract=off"],
    "reject.hip": ["-ffp-contract=off"],
}

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def _torch_lib_dir() -> str | None:
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec is None or spec.origin is None:
            return None
        d = os.path.join(os.path.dirname(spec.origin), "lib")
        return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None
    except Exception:
        return None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[-1]}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)

    def one(item):
        src, extra = item
        obj = os.path.join(OBJ, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES.items()))
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    tl = _torch_lib_dir()
    if tl:
        link += [f"-Wl,-rpath,{tl}"]
    if verbose:
        print(" ".join(link), flush=True)
    _run(link)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
