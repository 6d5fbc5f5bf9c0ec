"""Builds libditango.so in-tree with hipcc for gfx950.

Usage: python context_state_reuse_amd/build.py  (or __graft_entry__.build()).
Run it as a file: importing the package first would load the library.
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

SOURCES = ["host.cpp", "partial.hip", "merge.hip", "stats.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libditango.so)")


def _flags() -> list[str]:
    # -fno-honor-nans: from finite inputs no kernel makes a NaN (masked keys
    # score -FLT_MAX rather than -inf and every softmax row holds at least one
    # key), so NaN handling is dead code; without the flag every max of MFMA
    # results is preceded by a NaN-quieting canonicalize.  Inputs that hold
    # NaN or infinity give unspecified outputs.
    # -amdgpu-mfma-vgpr-form: MFMA results land in VGPRs, where the softmax
    # reads them, instead of AGPRs that need copies.
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-result"]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def _check_kernel_stubs(path: str) -> None:
    """The host pass can drop a kernel's launch stub without a diagnostic
    (device code it cannot compile for the host); the library would then
    fail to load.  Reject it here with the kernels named."""
    nm = shutil.which("nm")
    if nm is None:
        return
    r = subprocess.run([nm, "-D", "-C", "--undefined-only", path], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True)
    missing = [ln.split("U", 1)[-1].strip() for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(path)
        raise RuntimeError("kernel launch stubs missing from the host code:\n  " + "\n  ".join(missing))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link `out`.  `defines` (e.g. ["X=1"]) build
    a variant library for side-by-side measurement."""
    hipcc = _hipcc()
    objdir = OBJDIR if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        # the host half checks for NaN (scales, planner drifts): no
        # -fno-honor-nans there
        flags = _flags() if src.endswith(".hip") else [f for f in _flags() if f != "-fno-honor-nans"]
        jobs.append(([hipcc, *flags, *dflags, *lang, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, cmd) for cmd, _ in jobs]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[o for _, o in jobs]])
    _check_kernel_stubs(tmp)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
