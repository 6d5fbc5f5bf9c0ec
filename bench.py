"""Benchmark of partitioned attention with selective state reuse on one MI355X.

One step = one denoising step of one attention layer through the whole hot
path: build the step's selection mask, fresh partial attention for every
COMPUTE pair (states written into the cache), cache metadata update, and the
LSE-weighted merge of all P states per row.  The partial attention and the
merge run as one fused launch (ditango_step; with --group,
ditango_group_attn_partial_merge); --separate runs them as two launches
(ditango_attn_partial or ditango_group_attn_partial, then the merge) and
times each.  Inputs of every step are
resident in HBM before timing; the anchor step (all fresh) runs untimed first,
then warm-up and timed steps cycle over the workload's steady-state steps
t = 1 .. steps-1 with their masks.

Prints one JSON line.  value = effective (dense-equivalent) attention
TFLOP/s = 4 N^2 d H / time per step, so reuse can lift it above what the
fresh work alone would run at.  "roofline" describes the dominant kernel,
timed with HIP events on the stream it runs on; "cpu_baseline" times the fp64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "effective attention TFLOP/s and ms/denoise-step at given reuse ratio, 1 GPU"
DEFAULT_WORKLOAD = "long"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40, help="timed steps")
    ap.add_argument("--warmup", type=int, default=8, help="untimed steady-state steps after the anchor")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="image | video_100 | video_50 | video_25 | long | stress | tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-steps", type=int, default=0, help="timed steady-state steps of the oracle sample (0: auto, about 12 s)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--group", type=int, default=0,
                    help="run the grouped, composed state cache with this group size (0: per-pair cache)")
    ap.add_argument("--compose", type=int, default=0,
                    help="with --group: after the timed steps, time one merge of groups by this factor")
    ap.add_argument("--window-residual", action="store_true",
                    help="window attention with residual sharing: the anchor step computes every pair and caches "
                         "full-minus-window outputs; steady steps compute the window pairs (nearest partitions) only")
    ap.add_argument("--state-dtype", choices=("fp32", "bf16"), default="fp32",
                    help="number format of the cached states' OUT (fp32: the default; bf16 halves the cache)")
    ap.add_argument("--separate", action="store_true",
                    help="partial attention and merge as two launches instead of the fused step (both caches)")
    ap.add_argument("--planner", action="store_true",
                    help="anchor-guided planner picks each step's mask (per-pair cache); extra measurement")
    ap.add_argument("--plan-steps", type=int, default=16, help="denoising steps of the planned run")
    ap.add_argument("--plan-group", type=int, default=2, help="planner group size g")
    ap.add_argument("--plan-reuse", type=float, default=0.75, help="planner target reuse fraction")
    ap.add_argument("--plan-drift", type=float, default=0.1, help="planner anchor drift bound")
    ap.add_argument("--group-masks", choices=("nearest", "workload"), default="nearest",
                    help="with --group: group-aligned masks (local pair plus the nearest groups, as many "
                         "fresh partitions per row as the workload's masks) or the workload's own pair masks")
    return ap.parse_args()


def fresh_flops(w, mask) -> float:
    """4 * len_q * len_k * d per fresh pair and head (QK^T and PV)."""
    lens = np.array([min(w.S, w.N - p * w.S) for p in range(w.P)], dtype=np.float64)
    return float(4.0 * w.d * w.H * (np.outer(lens, lens) * mask).sum())


def token_reuse(w, fresh: float) -> float:
    """Reuse weighted by work: the share of the step's 4*N^2*d*H dense score
    FLOPs not computed fresh (equals the pair share unless partitions differ
    in length)."""
    return 1.0 - fresh / (4.0 * w.N * w.N * w.d * w.H)


def state_row_bytes(d: int, bf16: bool = False) -> int:
    """One cached state row: d OUT values (fp32, or bf16) and an fp32 LSE."""
    return (2 if bf16 else 4) * d + 4


def out_row_bytes(d: int) -> int:
    """One composed output row: d fp32 OUT values and an fp32 LSE."""
    return 4 * d + 4


def merge_bytes(w, bf16: bool = False) -> float:
    """Per row and head: read P cached states, write one fp32 output row."""
    return float(w.H * w.N * (w.P * state_row_bytes(w.d, bf16) + out_row_bytes(w.d)))


def state_store_bytes(w, mask, bf16: bool = False) -> float:
    lens = np.array([min(w.S, w.N - p * w.S) for p in range(w.P)], dtype=np.float64)
    return float(w.H * state_row_bytes(w.d, bf16) * (lens[:, None] * mask).sum())


def group_work(w, g, computed, bf16: bool = False):
    """Fresh FLOPs (4 * len_q * keys * d per computed slot and head) and
    merge bytes (the live slots' state rows read plus one output row written
    per row and head) of one grouped step."""
    from context_state_reuse_amd import group_slot_keys, group_slot_live
    lens = [min(w.S, w.N - q * w.S) for q in range(w.P)]
    ns = computed.shape[1]
    flops = sum(4.0 * w.d * w.H * lens[q] * group_slot_keys(w.N, w.P, g, q, s)
                for q in range(w.P) for s in range(ns) if computed[q, s])
    live = [sum(1 for s in range(ns) if group_slot_live(w.P, g, q, s)) for q in range(w.P)]
    mbytes = sum(float(w.H * lens[q] * (live[q] * state_row_bytes(w.d, bf16) + out_row_bytes(w.d)))
                 for q in range(w.P))
    return flops, mbytes


def source_hash(*names) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so a
    stored counter run stays matched to its code across comment edits."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "context_state_reuse_amd", "csrc", n)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("- ") and ":" in ln:
                k, v = ln[2:].split(":", 1)
                rec[k.strip()] = v.strip().strip("`")
    if rec.get("kernel_source_sha") != src_hash:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


BLAS_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")
ORACLE_CORE_FLOPS = 4.5e10    # fp64 oracle FLOP/s per core, single-threaded BLAS (measured on a 16-core EPYC host, long sample)
MAX_ORACLE_WORKERS = 16       # the host share of one GPU


def _oracle_worker(conn, wname: str, heads: list, stride: int) -> None:
    """One oracle process: its heads, every `stride`-th query row, stepped by
    the parent (inputs and mask prepared untimed, then the step on "go")."""
    import synth
    from oracle.masks import step_mask
    from oracle.reuse import StateReuseOracle
    w = synth.get(wname)
    rows = None if stride == 1 else np.arange(0, w.N, stride)
    orc = StateReuseOracle(w.N, w.P, w.d, rows=rows)
    stream = synth.InputStream(w, heads)
    while True:
        msg = conn.recv()
        if msg is None:
            break
        t, tt = msg
        if t == 0 or tt > stream.t:
            qb, kb, vb = stream.next()
        inp = {h: (synth.bf16_bits_to_f64(qb[i]), synth.bf16_bits_to_f64(kb[i]), synth.bf16_bits_to_f64(vb[i]))
               for i, h in enumerate(heads)}
        mask = step_mask(w, tt)
        conn.send("ready")
        conn.recv()
        orc.step(t, mask, inp)
        conn.send("done")
    conn.close()


def cpu_baseline(w, fresh_per_step: float, target_s: float = 15.0, steps: int = 0):
    """The fp64 oracle on the host cores, one process per core with
    single-threaded BLAS, heads spread over the processes, stepped in lock-step
    by this process: an untimed anchor step (all fresh), then timed
    steady-state steps cycling over t = 1 .. steps-1.  The sample is one head
    per process and every r-th query row (the oracle's own row subset, exact
    for those rows), r chosen so that about `target_s` seconds are timed.
    Run before the GPU is touched: the workers are started as fresh
    interpreters."""
    import multiprocessing as mp
    cores = max(1, min(MAX_ORACLE_WORKERS, len(os.sched_getaffinity(0)), w.H))
    heads = list(range(cores))
    per_head_step = fresh_per_step / w.H                  # FLOP, all rows
    n_steps = steps or 3
    stride = max(1, int(np.ceil(per_head_step * n_steps / (ORACLE_CORE_FLOPS * target_s))))
    if stride == 1 and not steps:
        n_steps = int(min(12, max(3, target_s * ORACLE_CORE_FLOPS / max(per_head_step, 1.0))))
    ctx = mp.get_context("spawn")
    saved = {k: os.environ.get(k) for k in BLAS_THREAD_VARS}
    for k in BLAS_THREAD_VARS:
        os.environ[k] = "1"
    procs, conns = [], []
    try:
        for h in heads:
            a, b = ctx.Pipe()
            p = ctx.Process(target=_oracle_worker, args=(b, w.name, [h], stride), daemon=True)
            p.start()
            procs.append(p)
            conns.append(a)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    timed, times = 0.0, []
    try:
        for t in range(1 + n_steps):
            tt = 1 + (t - 1) % max(w.steps - 1, 1) if t else 0
            for c in conns:
                c.send((t, tt))
            for c in conns:
                assert c.recv() == "ready"
            t0 = time.perf_counter()
            for c in conns:
                c.send("go")
            for c in conns:
                assert c.recv() == "done"
            if t:
                times.append(time.perf_counter() - t0)
        timed = float(sum(times))
    finally:
        for c in conns:
            try:
                c.send(None)
            except (BrokenPipeError, OSError):
                pass
        for p in procs:
            p.join(timeout=30)
    n_rows = len(range(0, w.N, stride))
    dense = 4.0 * n_rows * w.N * w.d * len(heads)         # dense-equivalent FLOPs of one sample step
    return {"value": dense * len(times) / timed / 1e12, "unit": "TFLOP/s", "cores": len(procs), "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": host_cpu_model(),
            "ms_per_sample_step": round(1e3 * timed / len(times), 1),
            "sample": f"{w.name}: {len(procs)} processes (single-threaded BLAS), one head each ({len(heads)} of "
                      f"{w.H} heads), {'every query row' if stride == 1 else f'every {stride}th query row'} ({n_rows} of {w.N}); an untimed all-fresh anchor "
                      f"step, then {len(times)} steady-state steps timed in lock-step, {timed:.1f} s; fp64 NumPy "
                      f"oracle; effective TFLOP/s counts 4*rows*N*d per sampled head and step"}


def planner_run(args, w, lib, torch, dev):
    """Steps chosen by the anchor-guided planner (per-pair cache), timed per
    phase with host synchronisation (the planner reads the statistics on the
    host): local pairs + their signatures, planning, the other chosen pairs
    + t_c + merge, and the statistics fed back.  Every step is timed, the
    two warm-up anchors included."""
    import synth
    w = w.scaled(steps=args.plan_steps)
    stream = synth.InputStream(w)
    qkv = [tuple(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for b in stream.next())
           for _ in range(w.steps)]
    sd = args.state_dtype
    cache = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=sd)
    planner = lib.Planner(w.P, args.plan_group, w.H, args.plan_reuse, args.plan_drift)
    run = lib.PlannedSteps(cache, planner)
    dense = 4.0 * w.N * w.N * w.d * w.H
    # untimed: load every kernel once (first launches load code objects)
    warm = lib.PlannedSteps(lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=sd),
                            lib.Planner(w.P, args.plan_group, w.H, args.plan_reuse, args.plan_drift))
    for t in range(3):
        warm.step(t, *qkv[t])
    del warm
    masks, anchors, ms = [], [], []
    torch.cuda.synchronize()
    for t in range(w.steps):
        t0 = time.perf_counter()
        mask, anchor, _, _ = run.step(t, *qkv[t])
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t0) * 1e3)
        masks.append(mask)
        anchors.append(anchor)
    # the same steps with the planner's masks through the plain step path:
    # the planner's own cost is the difference
    cache2 = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=sd)
    torch.cuda.synchronize()
    ms_plain = []
    for t in range(w.steps):
        t0 = time.perf_counter()
        lib.ditango_step(*qkv[t], masks[t], t, cache2)
        torch.cuda.synchronize()
        ms_plain.append((time.perf_counter() - t0) * 1e3)
    sel = [i for i, a in enumerate(anchors) if not a]
    ms_step = float(np.mean(ms))
    out = {
        "metric": METRIC, "value": round(dense / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": w.steps, "warmup": 0, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.F}x{w.Hh}x{w.W} = {w.N} tokens, H={w.H}, d={w.d}, P={w.P}, "
                               f"{w.steps} steps, masks from the anchor-guided planner (g={args.plan_group}, "
                               f"target reuse {args.plan_reuse}, drift bound {args.plan_drift})",
                   "tokens": w.N, "heads": w.H, "head_dim": w.d, "partitions": w.P,
                   "reuse_ratio": round(1.0 - float(np.mean([m.mean() for m in masks])), 4),
                   "parallelism": "none (all partitions on one GPU)",
                   **({"inputs": f"specified {w.dtype}: the library computes on bf16 copies of the {w.dtype} "
                                 f"inputs (error against the fp64 oracle on the unrounded inputs: "
                                 f"tests/test_gpu_parity.py::test_tiny_fp32_masters_error)"}
                      if w.dtype != "bf16" else {})},
        "planner": {"anchor_steps": [i for i, a in enumerate(anchors) if a],
                    "reuse_selective_steps": round(1.0 - float(np.mean([masks[i].mean() for i in sel])), 4) if sel else None,
                    "ms_per_step_planned": round(ms_step, 4),
                    "ms_per_step_same_masks_plain": round(float(np.mean(ms_plain)), 4),
                    "ms_planned_each": [round(x, 3) for x in ms], "ms_plain_each": [round(x, 3) for x in ms_plain],
                    "eps": planner.eps},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the path runs all P partitions on one device and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    # The oracle's timing runs first, before anything touches the GPU: its
    # worker processes start as fresh interpreters.
    cpu_rec = None
    if not (args.no_cpu_baseline or args.group or args.window_residual or args.planner):
        import synth
        from oracle.masks import step_mask
        w0 = synth.get(args.workload)
        fresh0 = float(np.mean([fresh_flops(w0, step_mask(w0, t)) for t in (range(1, w0.steps) or [0])]))
        cpu_rec = cpu_baseline(w0, fresh0, steps=args.cpu_steps)

    import torch

    import context_state_reuse_amd as lib
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.get(args.workload)
    bf16 = args.state_dtype == "bf16"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.planner:
        planner_run(args, w, lib, torch, dev)
        return

    # ---- inputs of every step resident in HBM
    stream = synth.InputStream(w)
    qkv = []
    for t in range(w.steps):
        bits = stream.next()
        qkv.append(tuple(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for b in bits))
    del stream
    g = args.group
    if g:
        cache = lib.GroupedStateCache(w.H, w.N, w.d, w.P, g, state_dtype=args.state_dtype)
        cache_bytes = cache.device_bytes
    else:
        cache = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=args.state_dtype)
        cache_bytes = sum(lib.ditango_states_bytes(cache.shape))
    O = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device=dev)
    LSE = torch.empty((w.H, w.N), dtype=torch.float32, device=dev)

    step_no = [0]
    computed_log = []
    n_groups = max(1, round(w.n_fresh / g)) if g else 0
    wr = args.window_residual
    if wr and g:
        print("--window-residual works on the per-pair cache; drop --group", file=sys.stderr)
        sys.exit(2)
    if wr:
        wmask = lib.ditango_mask_build("radius", w.P, 1) if w.policy == "radius" else \
            lib.ditango_mask_build("nearest", w.P, min(w.n_fresh, w.P))
        R = torch.empty((w.H, w.N, w.d), dtype=torch.float32, device=dev)
        mask_of = lambda t: lib.ditango_mask_build("all", w.P) if t == 0 else wmask
        mask_desc = f"window residual, window = {'radius-1' if w.policy == 'radius' else 'nearest-' + str(w.n_fresh)}"
    elif g and args.group_masks == "nearest":
        gmask = lib.ditango_group_mask_build(w.P, g, n_groups)
        mask_of = lambda t: lib.ditango_mask_build("all", w.P) if t == 0 else gmask
        mask_desc = f"local pair + {n_groups} nearest group(s) of {g}"
    else:
        mask_of = lambda t: lib.workload_mask(w, t)
        mask_desc = f"{w.policy}-{w.n_fresh}"

    fused = not (wr or args.separate)

    def step(t: int, events=None):
        mask = mask_of(t)
        Q, K, V = qkv[t]
        if events is not None:
            events[0].record()
        if fused:
            if g:
                lib.ditango_group_attn_partial_merge(Q, K, V, mask, cache, O, LSE)
                computed = lib.ditango_group_cache_update(cache, mask, step_no[0])
                if events is not None:
                    computed_log.append(computed)
            else:
                lib.ditango_step(Q, K, V, mask, step_no[0], cache, O, LSE)
            if events is not None:
                events[1].record()
                events[2].record()
            step_no[0] += 1
            return mask
        if g:
            lib.ditango_group_attn_partial(Q, K, V, mask, cache)
        else:
            lib.ditango_attn_partial(Q, K, V, mask, cache)
        if events is not None:
            events[1].record()
        if g:
            computed = lib.ditango_group_cache_update(cache, mask, step_no[0])
            lib.ditango_group_merge(cache, O, LSE)
            if events is not None:
                computed_log.append(computed)
        elif wr:
            lib.ditango_state_cache_update(cache, mask, step_no[0])
            lib.ditango_window_residual_merge(cache, wmask, lib.DITANGO_WR_FULL if t == 0 else lib.DITANGO_WR_WINDOW,
                                              R, O, LSE)
        else:
            lib.ditango_state_cache_update(cache, mask, step_no[0])
            lib.ditango_state_merge(cache, O, LSE)
        if events is not None:
            events[2].record()
        step_no[0] += 1
        return mask

    if args.calibrate_copy:
        # plain device copy of 1 GiB: 1 GiB read + 1 GiB written
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    steady = list(range(1, w.steps)) or [0]
    step(0)                                         # anchor: all fresh
    for i in range(args.warmup):
        step(steady[i % len(steady)])
    # one more anchor step (all fresh, inputs of step 0), timed on its own and
    # reported apart from the steady-state steps; the cache it leaves is the
    # one the first anchor left
    anchor_ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    step(0, anchor_ev)
    if g:
        computed_log.pop()
    torch.cuda.synchronize()
    anchor_rec = {"ms": round(anchor_ev[0].elapsed_time(anchor_ev[2]), 4)}
    if not fused:
        anchor_rec.update(partial_ms=round(anchor_ev[0].elapsed_time(anchor_ev[1]), 4),
                          merge_ms=round(anchor_ev[1].elapsed_time(anchor_ev[2]), 4))

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    masks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        masks.append(step(steady[i % len(steady)], evs[i]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_step = elapsed * 1e3 / args.steps
    t_partial = np.mean([e[0].elapsed_time(e[1]) for e in evs])      # ms
    t_merge = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    dense = 4.0 * w.N * w.N * w.d * w.H
    value = dense / (ms_step * 1e-3) / 1e12
    if g:
        work = [group_work(w, g, c, bf16) for c in computed_log]
        fresh = np.mean([f for f, _ in work])
        mb = np.mean([b for _, b in work])
        lens = np.array([min(w.S, w.N - p * w.S) for p in range(w.P)], dtype=np.float64)
        sb = np.mean([w.H * state_row_bytes(w.d, bf16) * (lens[:, None] * c).sum() for c in computed_log])
        reuse = 1.0 - np.mean([c.sum() / sum(lib.group_slot_live(w.P, g, q, s) for q in range(w.P)
                                              for s in range(c.shape[1])) for c in computed_log])
    else:
        fresh = np.mean([fresh_flops(w, m) for m in masks])
        reuse = 1.0 - np.mean([m.mean() for m in masks])
        mb = merge_bytes(w, bf16)
        sb = np.mean([state_store_bytes(w, m, bf16) for m in masks])
        if wr:
            # window step: the window states and the residual read, one output written
            lens = np.array([min(w.S, w.N - p * w.S) for p in range(w.P)], dtype=np.float64)
            mb = float(w.H * (lens * (wmask.sum(axis=1) * state_row_bytes(w.d, bf16) + 4 * w.d
                                      + out_row_bytes(w.d))).sum())

    partial_tflops = fresh / (t_partial * 1e-3) / 1e12
    merge_gbs = mb / (t_merge * 1e-3) / 1e9 if t_merge > 0 else 0.0
    src = source_hash("partial.hip")
    cache_desc = (f"grouped, g={g}: {cache.n_slots} slots per query partition" if g
                  else "per pair: P slots per query partition")
    compose_rec = None
    if g and args.compose:
        # one in-place merge of groups by args.compose; bytes: every live old
        # group state read once, every new group state written once
        k = args.compose
        lens = [min(w.S, w.N - q * w.S) for q in range(w.P)]
        m_old, g_new = cache.n_slots - 1, g * k
        m_new = lib.ditango_group_slots(w.P, g_new) - 1
        cbytes = 0.0
        for q in range(w.P):
            for i in range(m_new):
                parts = sum(lib.group_slot_live(w.P, g, q, 1 + j) for j in range(k * i, min(k * i + k, m_old)))
                cbytes += (parts + (1 if parts else 0)) * float(w.H * lens[q] * state_row_bytes(w.d, bf16))
        before = cache.device_bytes
        # the first launch of a kernel in a process pays a one-time load: merge
        # the groups of a one-token-per-partition cache of the same P, g, d and
        # state format first (same kernel instantiation), untimed
        warm = lib.GroupedStateCache(1, w.P, w.d, w.P, g, state_dtype=args.state_dtype)
        wq = torch.zeros((1, w.P, w.d), dtype=torch.bfloat16, device=dev)
        every = np.ones((w.P, w.P), np.uint8)
        lib.ditango_group_attn_partial(wq, wq, wq, every, warm)
        lib.ditango_group_cache_update(warm, every, 0)
        warm.compose(k)
        del warm, wq
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        cache.compose(k, after=ev[1].record)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        compose_rec = {"factor": k, "group_size_from": g, "group_size_to": g_new, "ms": round(ms, 4),
                       "bytes": cbytes, "gbs": round(cbytes / (ms * 1e-3) / 1e9, 1),
                       "cache_bytes_before": before, "cache_bytes_after": cache.device_bytes}

    if fused:
        roof = {"kernel": "group_step_kernel" if g else "step_kernel", "bound": "mfma",
                "achieved": round(partial_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(partial_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None if (g or bf16) else stored_traffic("step", w.name, src),
                "avg_launch_ms": round(float(t_partial), 4),
                "algorithmic_per_launch": f"{fresh:.4e} FLOP (4*len_q*len_k*d per fresh "
                                          f"{'slot, len_k = keys of its members' if g else 'pair'} and head); the "
                                          f"same launch moves {mb + sb:.4e} B of states "
                                          f"({'live slots' if g else 'P'}*({2 if bf16 else 4}d+4) read + (4d+4) written per row and "
                                          f"head, {2 if bf16 else 4}d+4 per fresh {'slot' if g else 'pair'} row stored)"}
    elif t_partial >= t_merge:
        roof = {"kernel": "partial_kernel", "bound": "mfma", "achieved": round(partial_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(partial_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None if (g or wr or bf16) else stored_traffic("partial", w.name, src),
                "avg_launch_ms": round(float(t_partial), 4),
                "algorithmic_per_launch": f"{fresh:.4e} FLOP (4*len_q*len_k*d per fresh "
                                          f"{'slot, len_k = keys of its members' if g else 'pair'} and head)"}
    else:
        roof = {"kernel": "merge_kernel", "bound": "hbm", "achieved": round(merge_gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(merge_gbs / PEAK_HBM_GBS, 4),
                "traffic": None if (g or wr or bf16) else stored_traffic("merge", w.name, source_hash("merge.hip")),
                "avg_launch_ms": round(float(t_merge), 4),
                "algorithmic_per_launch": f"{mb:.4e} B ({'live slots' if g else 'P'}*({2 if bf16 else 4}d+4) read + (4d+4) "
                                          f"written per row and head)"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.F}x{w.Hh}x{w.W} = {w.N} tokens, H={w.H}, d={w.d}, P={w.P}, "
                               f"{mask_desc} mask", "tokens": w.N, "heads": w.H, "head_dim": w.d,
                   "partitions": w.P, "reuse_ratio": round(float(reuse), 4),
                   "reuse_ratio_tokens": round(token_reuse(w, float(fresh)), 4),
                   "state_cache": ("per pair, window states only, plus a residual [H][N][d]" if wr else cache_desc),
                   "state_dtype": f"OUT {args.state_dtype}, LSE fp32",
                   "cache_bytes": cache_bytes,
                   "fresh_pairs_per_step": float(np.mean([m.sum() for m in masks])),
                   **({"computed_slots_per_step": float(np.mean([c.sum() for c in computed_log]))} if g else {}),
                   "parallelism": "none (all partitions on one GPU)",
                   **({"inputs": f"specified {w.dtype}: the library computes on bf16 copies of the {w.dtype} "
                                 f"inputs (error against the fp64 oracle on the unrounded inputs: "
                                 f"tests/test_gpu_parity.py::test_tiny_fp32_masters_error)"}
                      if w.dtype != "bf16" else {})},
        "roofline": roof,
        "kernels": ({
            "step": {"ms": round(float(t_partial), 4), "tflops": round(partial_tflops, 2),
                     "mfma_frac": round(partial_tflops / PEAK_BF16_TFLOPS, 4), "fresh_flop": fresh,
                     "state_bytes": float(mb + sb),
                     "gbs": round((mb + sb) / (t_partial * 1e-3) / 1e9, 1),
                     "hbm_frac": round((mb + sb) / (t_partial * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     # the fresh FLOP at the MFMA peak plus the state bytes at the HBM peak, over
                     # the launch: the bound when a block's composition cannot overlap its own
                     # matrix work (d = 128: a block fills its CU)
                     "serial_bound_frac": round((fresh / (PEAK_BF16_TFLOPS * 1e12) + (mb + sb) / (PEAK_HBM_GBS * 1e9))
                                                / (t_partial * 1e-3), 4)},
        } if fused else {
            "partial": {"ms": round(float(t_partial), 4), "tflops": round(partial_tflops, 2),
                        "mfma_frac": round(partial_tflops / PEAK_BF16_TFLOPS, 4), "fresh_flop": fresh,
                        "state_store_bytes": sb},
            "merge": {"ms": round(float(t_merge), 4), "gbs": round(merge_gbs, 1),
                      "hbm_frac": round(merge_gbs / PEAK_HBM_GBS, 4), "bytes": mb},
        }),
    }
    # HBM fraction of the whole step: the merge's bytes plus the fresh states
    # stored, over the step time
    out["step_hbm"] = {"bytes": float(mb + sb),
                       "frac": round((mb + sb) / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out["anchor_step"] = anchor_rec
    if compose_rec is not None:
        out["group_compose"] = compose_rec
    if cpu_rec is not None:
        out["cpu_baseline"] = cpu_rec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
