"""Build libpva.so (HIP kernels for gfx950 + host planner + C-ABI) in-tree,
and libpva_timeline.so, the same sources with the per-workgroup timeline
compiled in (PVA_WG_TIMELINE; for performance analysis only).

Usage: python -m packed_varlen_masked_attn_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpva.so")
BUILD_TIMELINE = os.path.join(ROOT, "_build", "timeline")
LIB_TIMELINE = os.path.join(PKG, "libpva_timeline.so")

SOURCES = ["plan.cpp", "api.cpp", "fwd_bf16.hip", "fwd_fp8.hip", "merge.hip", "noalloc.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# Packed FP32 instructions are kept out of every kernel (the compiler would
# otherwise form v_pk_* FP32 ops from plain float code).
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpva.so")


def _compile(src: str, verbose: bool, timeline: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_TIMELINE if timeline else BUILD, src + ".o")
    extra = ["-DPVA_WG_TIMELINE"] if timeline else []
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *COMMON, *extra, *DEVICE, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, *extra, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise))
    return obj


def _link(objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, timeline: bool = True) -> str:
    """Compile every source and link libpva.so next to this file (and, with
    `timeline`, libpva_timeline.so). Always rebuilds. Returns libpva.so."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES]
    if timeline:
        os.makedirs(BUILD_TIMELINE, exist_ok=True)
        jobs += [(s, True) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    if timeline:
        _link(objs[len(SOURCES):], LIB_TIMELINE, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
