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


def run_steps(w, masks=None, steps=None, on_step=None, label="", fused=False, state_dtype="fp32"):
    """Run the library over the steps of workload w.

    masks: optional {t: mask}; default is the library's own mask builder.
    fused: each step is one ditango_step call (the fused partial + merge
    launch) instead of partial, t_c update and merge called one by one.
    state_dtype: the cache's OUT format ("fp32" or "bf16").
    on_step(t, mask, reused, cache, O, LSE) is called after each step
    (after a device synchronisation).
    """
    import torch

    import context_state_reuse_amd as lib

    n = w.steps if steps is None else steps
    cache = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    O = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    LSE = torch.empty((w.H, w.N), dtype=torch.float32, device="cuda")
    for t in range(n):
        t0 = time.time()
        qb, kb, vb = stream.next()
        Q, K, V = to_device(qb), to_device(kb), to_device(vb)
        del qb, kb, vb
        mask = lib.workload_mask(w, t) if masks is None or t not in masks else np.asarray(masks[t], np.uint8)
        if fused:
            _, _, reused = lib.ditango_step(Q, K, V, mask, t, cache, O, LSE)
        else:
            lib.ditango_attn_partial(Q, K, V, mask, cache)
            reused = lib.ditango_state_cache_update(cache, mask, t)
            lib.ditango_state_merge(cache, O, LSE)
        torch.cuda.synchronize()
        log(f"  [{label or w.name}{' fused' if fused else ''} {state_dtype}] step {t}: fresh {int(mask.sum())}/{w.P * w.P} pairs, {time.time() - t0:.1f}s")
        if on_step is not None:
            on_step(t, mask, reused, cache, O, LSE)
        del Q, K, V
    return cache


def run_group_steps(w, g, masks=None, steps=None, compose_at=None, on_step=None, label="", budget_at=None,
                    fused=False, state_dtype="fp32"):
    """Run the grouped-cache path of the library over the steps of workload w.

    fused: the slots' fresh states and the composition in one launch
    (ditango_group_attn_partial_merge), then the t_c update, instead of
    partial, t_c update and merge one by one.
    state_dtype: the slots' OUT format ("fp32" or "bf16").

    compose_at: optional {t: k}: merge groups by k right before step t.
    budget_at: optional {t: bytes}: right before step t, merge groups by 2
    while the cache exceeds that many bytes (the memory trigger).
    on_step(t, mask, computed, cache, O, LSE) is called after each step.
    """
    import torch

    import context_state_reuse_amd as lib

    n = w.steps if steps is None else steps
    cache = lib.GroupedStateCache(w.H, w.N, w.d, w.P, g, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    O = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    LSE = torch.empty((w.H, w.N), dtype=torch.float32, device="cuda")
    for t in range(n):
        t0 = time.time()
        qb, kb, vb = stream.next()
        Q, K, V = to_device(qb), to_device(kb), to_device(vb)
        del qb, kb, vb
        if compose_at and t in compose_at:
            cache.compose(compose_at[t])
            log(f"  [{label or w.name}] before step {t}: groups merged to g={cache.g}, {cache.n_slots} slots")
        if budget_at and t in budget_at:
            merges = cache.fit(budget_at[t], 2)
            log(f"  [{label or w.name}] before step {t}: budget {budget_at[t]} B, {merges} merge(s), g={cache.g}, "
                f"{cache.device_bytes} B")
        mask = lib.workload_mask(w, t) if masks is None or t not in masks else np.asarray(masks[t], np.uint8)
        if fused:
            lib.ditango_group_attn_partial_merge(Q, K, V, mask, cache, O, LSE)
            computed = lib.ditango_group_cache_update(cache, mask, t)
        else:
            lib.ditango_group_attn_partial(Q, K, V, mask, cache)
            computed = lib.ditango_group_cache_update(cache, mask, t)
            lib.ditango_group_merge(cache, O, LSE)
        torch.cuda.synchronize()
        log(f"  [{label or w.name}{' fused' if fused else ''} {state_dtype}] step {t}: g={cache.g}, {int(computed.sum())} slots computed, "
            f"{time.time() - t0:.1f}s")
        if on_step is not None:
            on_step(t, mask, computed, cache, O, LSE)
        del Q, K, V
    return cache


def run_window_residual_steps(w, window, steps=None, on_step=None, label="", state_dtype="fp32"):
    """Window attention with residual sharing through the library: step 0
    computes every pair and caches the residual, later steps compute the
    window pairs only.  on_step(t, cache, R, O, LSE) after each step."""
    import torch

    import context_state_reuse_amd as lib

    n = w.steps if steps is None else steps
    cache = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    R = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    O = torch.empty_like(R)
    LSE = torch.empty((w.H, w.N), dtype=torch.float32, device="cuda")
    window = np.asarray(window, np.uint8)
    for t in range(n):
        t0 = time.time()
        qb, kb, vb = stream.next()
        Q, K, V = to_device(qb), to_device(kb), to_device(vb)
        mask = np.ones((w.P, w.P), np.uint8) if t == 0 else window
        lib.ditango_attn_partial(Q, K, V, mask, cache)
        lib.ditango_state_cache_update(cache, mask, t)
        lib.ditango_window_residual_merge(cache, window, lib.DITANGO_WR_FULL if t == 0 else lib.DITANGO_WR_WINDOW,
                                          R, O, LSE)
        torch.cuda.synchronize()
        log(f"  [{label or w.name}] window-residual step {t}: {time.time() - t0:.1f}s")
        if on_step is not None:
            on_step(t, cache, R, O, LSE)
        del Q, K, V
    return cache
