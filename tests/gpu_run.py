"""Drives the HIP path over a workload for the GPU tests (no oracle code here)."""
from __future__ import annotations

import sys
import time

import numpy as np

import synth


def log(*a):
    print(*a, flush=True, file=sys.stderr)


def to_device(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def run_steps(w, masks=None, steps=None, on_step=None, label=""):
    """Run the library over the steps of workload w.

    masks: optional {t: mask}; default is the library's own mask builder.
    on_step(t, mask, reused, cache, O, LSE) is called after each step
    (after a device synchronisation).
    """
    import torch

    import context_state_reuse_amd as lib

    n = w.steps if steps is None else steps
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    stream = synth.InputStream(w)
    O = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    LSE = torch.empty((w.H, w.N), dtype=torch.float32, device="cuda")
    for t in range(n):
        t0 = time.time()
        qb, kb, vb = stream.next()
        Q, K, V = to_device(qb), to_device(kb), to_device(vb)
        del qb, kb, vb
        mask = lib.workload_mask(w, t) if masks is None or t not in masks else np.asarray(masks[t], np.uint8)
        lib.ditango_attn_partial(Q, K, V, mask, cache)
        reused = lib.ditango_state_cache_update(cache, mask, t)
        lib.ditango_state_merge(cache, O, LSE)
        torch.cuda.synchronize()
        log(f"  [{label or w.name}] step {t}: fresh {int(mask.sum())}/{w.P * w.P} pairs, {time.time() - t0:.1f}s")
        if on_step is not None:
            on_step(t, mask, reused, cache, O, LSE)
        del Q, K, V
    return cache
