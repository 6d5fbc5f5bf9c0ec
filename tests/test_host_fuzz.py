"""The library's host half under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

host.cpp is compiled for the CPU with the four kernel launchers replaced by
stubs (tests/host_fuzz/stubs.cpp) that check every launch's parameters
against the kernels' limits (work-list sizes, pair and slot ids, grid size,
live-state masks) instead of launching.  A seeded driver
(tests/host_fuzz/fuzz.cpp) calls every entry point with valid, edge and
invalid arguments: mask builders over all policies and sizes, planner
sequences with NaN, infinite and zero statistics, per-pair and grouped
caches with random masks, steps, merges of groups and resets.  Any memory
error, undefined behaviour or broken launch contract fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
HERE = os.path.join(ROOT, "tests", "host_fuzz")


def _sanitizers_available() -> bool:
    return os.path.exists(CLANG) and bool(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan*x86_64*"))


@pytest.mark.skipif(not _sanitizers_available(), reason="ROCm clang++ with sanitizer runtimes not present")
def test_host_logic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_fuzz")
    cmd = [CLANG, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "context_state_reuse_amd", "csrc"),
           "-x", "c++", os.path.join(ROOT, "context_state_reuse_amd", "csrc", "host.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "fuzz.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stdout + b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    # every launcher was reached, so the contracts were exercised
    fields = r.stdout.split()
    kinds = ("fused_step", "group_step", "partial", "merge", "stats", "drift")
    launches = {fields[i]: int(fields[i + 1]) for i in range(len(fields) - 1) if fields[i] in kinds}
    assert len(launches) == len(kinds) and min(launches.values()) > 100, r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
