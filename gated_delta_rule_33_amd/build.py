"""Build the HIP library for gfx950 (hipcc, in-tree): libkda.so, and
libkda_debug.so, the same sources with KDA_DEBUG_CHECKS (device checks of
input preconditions, reported through the workspace flags).

Every HIP source is compiled with packed fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
DEBUG_LIB = os.path.join(PKG, "libkda_debug.so")
SOURCES = ["kda_api.cpp", "kda_prep.hip", "kda_intra.hip", "kda_fused.hip", "kda_recur.hip", "kda_layer.hip",
           "kda_cp.hip", "kda_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         "-Wno-unused-function"]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.basename(src) + ".o")
    extra = ["-DKDA_DEBUG_CHECKS=1"] if debug else []
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 4, debug: bool = False) -> str:
    """Build libkda.so (or, with debug, libkda_debug.so); returns its path."""
    os.makedirs(os.path.join(BUILD, "debug" if debug else ""), exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    lib = DEBUG_LIB if debug else LIB
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build_all(jobs: int = 4) -> list:
    return [build(jobs), build(jobs, debug=True)]


if __name__ == "__main__":
    print(build_all())
