"""Builds libmoe.so (the HIP library behind include/moe.h) in-tree for gfx950.

    python -m sparse_mixture_experts_level_amd.build

Each source in csrc/ is compiled with hipcc into _build/, then linked into
sparse_mixture_experts_level_amd/libmoe.so.  Packed-fp32 instructions are turned
off for all device code.  The debug library libmoe_debug.so is linked beside it
from the same kernels and api.cpp compiled with MOE_DEBUG_CHECKS (host checks of
the device-side preconditions, which synchronise the stream).
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
LIB = os.path.join(PKG, "libmoe.so")
DEBUG_LIB = os.path.join(PKG, "libmoe_debug.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", src, "-o", obj,
           f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    api = [s for s in srcs if os.path.basename(s) == "api.cpp"]
    jobs = [(s, list(extra), "") for s in srcs] + [(s, list(extra) + ["-DMOE_DEBUG_CHECKS"], ".debug") for s in api]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    release = objs[:len(srcs)]
    debug = [o for s, o in zip(srcs, release) if s not in api] + objs[len(srcs):]
    _link(release, LIB)
    _link(debug, DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build()
