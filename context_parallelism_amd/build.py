"""Build libcpattn.so in-tree with hipcc for gfx950.

``python context_parallelism_amd/build.py`` (or ``build()``) compiles every
source under ``csrc/`` into ``_build/`` and links
``context_parallelism_amd/libcpattn.so``. Always recompiles: this is also the
"does it build" check.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcpattn.so")

# Plain C++ (no HIP headers): the planner and the host-only entry points.
HOST_SOURCES = ["plan.cpp", "workspace.cpp", "capi_host.cpp", "plan_check.cpp"]
# Compiled as HIP for gfx950.
DEVICE_SOURCES = ["capi.cpp", "gather.hip", "attn_bf16.hip", "attn_bwd.hip", "attn_bwd_generic.hip", "attn_f32.hip",
                  "lse_merge.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed-fp32 VALU instructions are switched off for the device code.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcpattn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    cmds, objs = [], []
    for src in HOST_SOURCES + DEVICE_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        dev = src in DEVICE_SOURCES
        flags = COMMON + (DEVICE_FLAGS if dev else [])
        lang = ["-x", "hip"] if dev else ["-x", "c++"]
        cmds.append([cc] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
