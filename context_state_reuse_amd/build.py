"""Builds libditango.so in-tree with hipcc for gfx950.

Usage: python -m context_state_reuse_amd.build  (or __graft_entry__.build()).
Always recompiles.  Flags: -O3, C++17, gfx950 only, and packed fp32 VALU
instructions disabled (the kernels are written for scalar fp32 VALU).
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libditango.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["host.cpp", "partial.hip", "merge.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libditango.so)")


def _flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result"]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append(([hipcc, *_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, cmd) for cmd, _ in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[o for _, o in jobs]])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
