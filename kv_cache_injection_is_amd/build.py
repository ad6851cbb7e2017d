"""Builds libinferscale.so (HIP kernels + C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(PKG, "libinferscale.so")
HIPCC = "/opt/rocm/bin/hipcc"

SOURCES = ["abi.hip", "inject.hip", "topk.hip", "compose.hip", "attend.hip", "ingest.hip", "plan.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}"]


def build(verbose: bool = False, out: str = SO, defines=()) -> str:
    """Compiles the library to `out`; `defines` are extra -D tuning knobs."""
    objs = []
    tag = os.path.basename(out).replace(".so", "")
    for src in SOURCES:
        obj = os.path.join(CSRC, f"{src}.{tag}.o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    _run([HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", out], verbose)
    for o in objs:
        os.remove(o)
    return out


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose:
        print(" ".join(cmd))
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    print(build(verbose=True))
