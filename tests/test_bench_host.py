"""bench.py's host-side contract (CPU): it refuses more than one GPU, and its
FLOP and byte accounting matches the workload definitions."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_fresh_flops_and_merge_bytes_image():
    w = synth.get("image")
    m = np.zeros((w.P, w.P), np.uint8)
    m[0, 0] = m[3, 4] = 1
    # every partition of the image workload holds S = 2048 tokens
    assert bench.fresh_flops(w, m) == 2 * 4.0 * 2048 * 2048 * 72 * 16
    # a cached state row: 72 fp32 + one fp32 LSE = 292 bytes (bf16 OUT: 148); an output row: 292 bytes
    assert bench.merge_bytes(w) == 16 * 16384 * 9 * 73 * 4
    assert bench.state_store_bytes(w, m) == 16 * 73 * 4 * 2 * 2048
    assert bench.merge_bytes(w, bf16=True) == 16 * 16384 * (8 * 148 + 292)
    assert bench.state_store_bytes(w, m, bf16=True) == 16 * 148 * 2 * 2048


def test_fresh_flops_ragged_stress():
    w = synth.get("stress")
    m = np.zeros((w.P, w.P), np.uint8)
    m[w.P - 1, w.P - 1] = 1          # the ragged last partition against itself
    last = w.N - (w.P - 1) * w.S
    assert last == 531 and bench.fresh_flops(w, m) == 4.0 * last * last * w.d * w.H


def test_group_accounting_at_group_size_one_is_per_pair():
    w = synth.get("tiny")
    from oracle.groups import group_decisions
    m = np.array([[1, 1, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1], [0, 0, 1, 1]], np.uint8)
    computed = group_decisions(m, 1)
    flops, mbytes = bench.group_work(w, 1, computed)
    assert flops == bench.fresh_flops(w, m)
    assert mbytes == bench.merge_bytes(w)


def test_token_weighted_reuse():
    # equal partitions: the work-weighted reuse is the pair share
    w = synth.get("image")
    m = np.zeros((w.P, w.P), np.uint8)
    np.fill_diagonal(m, 1)
    m[0, 1] = 1
    assert abs(bench.token_reuse(w, bench.fresh_flops(w, m)) - (1 - m.mean())) < 1e-12
    # stress: the ragged last partition (531 of 549 tokens) carries less work
    w = synth.get("stress")
    m = np.zeros((w.P, w.P), np.uint8)
    m[w.P - 1, w.P - 1] = 1
    lens = np.array([min(w.S, w.N - p * w.S) for p in range(w.P)], float)
    expect = 1 - lens[-1] ** 2 / w.N ** 2
    assert abs(bench.token_reuse(w, bench.fresh_flops(w, m)) - expect) < 1e-12
    assert bench.token_reuse(w, bench.fresh_flops(w, m)) > 1 - m.mean()


def test_host_cpu_model_is_named():
    assert isinstance(bench.host_cpu_model(), str) and bench.host_cpu_model()
