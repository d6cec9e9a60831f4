"""Build the gfx950 shared library ``libace_moe.so`` in-tree with hipcc.

Run ``python -m token_adaptive_expert_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles all sources.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libace_moe.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "route.hip", "dispatch.hip", "expert.hip", "combine.hip", "calibrate.hip", "tables.hip",
           "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc to build")


def _compile(src: str, objdir: str = OBJDIR, defines=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + HIPCC_FLAGS + [f"-D{d}" for d in defines] + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link ``out``.  ``defines`` (NAME=VALUE strings)
    override the kernels' compile-time tuning knobs."""
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
