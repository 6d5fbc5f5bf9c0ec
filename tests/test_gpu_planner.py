"""GPU parity of the planner's statistics and of planned steps.

* ditango_pair_stats against the oracle's importance and signatures, taken
  from the oracle's own cache of the same steps (reduced workloads, ragged
  partitions, the three head dims).  Bar: W abs <= 2e-3 (an LSE error of
  1e-3 in the slot and in the merged LSE moves exp(LSE_k - LSE) by at most
  about 2e-3 relative, and W <= 1); SIG max-abs <= 2e-2 and mean-abs <= 2e-3
  (a mean of OUT rows errs by at most OUT's bound).
* planned steps: the library's planner picks each step's mask on the GPU
  statistics; every mask keeps the local pairs and whole groups, and the
  outputs match the oracle run with the same masks to the per-pair bar.
"""
import math

import numpy as np
import pytest

import synth
from oracle.planner import group_members, pair_signature, pair_weights
from oracle.reuse import StateReuseOracle

from gpu_run import log, to_device

pytestmark = pytest.mark.gpu

TOL_W, TOL_SIG_MAX, TOL_SIG_MEAN = 2e-3, 2e-2, 2e-3
TOL_O_MAX, TOL_O_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


def _scaled(base, name, F, Hh, W, H, **kw):
    return synth.get(base).scaled(name=name, F=F, Hh=Hh, W=W, H=H, **kw)


CASES = [
    _scaled("image", "image_small", 1, 57, 97, 2),            # d=72, ragged last partition
    _scaled("video_25", "video25_small", 5, 21, 29, 2),       # d=128
    _scaled("stress", "stress_small", 5, 16, 27, 2),          # d=64, P=32
    _scaled("tiny", "one_token_last", 1, 3, 7, 2, P=5),       # N=21, S=5: last partition of 1 token
    _scaled("tiny", "single_partition", 1, 9, 13, 1, P=1),    # P=1: the local pair only
]


def _oracle_stats(w, orc_cache, merged_lse):
    """Expected W [H][P][P] and SIG [H][P][P][d] from the oracle's cache."""
    P, S = w.P, w.S
    W = np.zeros((w.H, P, P))
    SIG = np.zeros((w.H, P, P, w.d))
    for h in range(w.H):
        lm = [merged_lse[h][q * S:min((q + 1) * S, w.N)] for q in range(P)]
        ls = [[orc_cache[(h, q, k)][1] for k in range(P)] for q in range(P)]
        W[h] = pair_weights(ls, lm)
        for q in range(P):
            for k in range(P):
                SIG[h, q, k] = pair_signature(orc_cache[(h, q, k)][0])
    return W, SIG


STATS_CASES = [(w, "fp32") for w in CASES] + [(CASES[0], "bf16"), (CASES[2], "bf16")]


@pytest.mark.parametrize("w,state_dtype", STATS_CASES, ids=[f"{w.name}_{sd}" for w, sd in STATS_CASES])
def test_pair_stats_match_oracle(w, state_dtype):
    import torch

    import context_state_reuse_amd as lib
    steps = 3
    orc = StateReuseOracle(w.N, w.P, w.d)
    cache = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    ones = np.ones((w.P, w.P), np.uint8)
    SIG = torch.zeros((w.H, w.P, w.P, w.d), dtype=torch.float32, device="cuda")
    for t in range(steps):
        qb, kb, vb = stream.next()
        mask = lib.workload_mask(w, t)
        res = orc.step(t, mask, {h: (synth.bf16_bits_to_f64(qb[h]), synth.bf16_bits_to_f64(kb[h]),
                                     synth.bf16_bits_to_f64(vb[h])) for h in range(w.H)})
        O, LSE, _ = lib.ditango_step(to_device(qb), to_device(kb), to_device(vb), mask, t, cache)
        sel = ones if t == 0 else mask
        W, SIG = lib.ditango_pair_stats(cache, LSE, sel, SIG=SIG)
        torch.cuda.synchronize()
        We, SIGe = _oracle_stats(w, orc.cache, res["LSE"])
        Wg, Sg = W.cpu().numpy().astype(np.float64), SIG.cpu().numpy().astype(np.float64)
        werr = np.abs(Wg - We).max()
        serr = np.abs(Sg - SIGe)
        log(f"  [{w.name}] step {t}: W abs {werr:.2e}, SIG max {serr.max():.2e} mean {serr.mean():.2e}")
        assert werr <= TOL_W, f"{w.name} step {t}: W abs {werr:.3g}"
        assert serr.max() <= TOL_SIG_MAX and serr.mean() <= TOL_SIG_MEAN, f"{w.name} step {t}: SIG"
        np.testing.assert_allclose(Wg.sum(axis=2), 1.0, atol=1e-4)
        # signatures alone (no importance, selected pairs only): the same values
        _, SIG2 = lib.ditango_pair_stats(cache, None, sel, SIG=torch.full_like(SIG, 7.0), want_w=False)
        S2 = SIG2.cpu().numpy()
        assert np.array_equal(S2[:, sel == 1], SIG.cpu().numpy()[:, sel == 1])
        assert (S2[:, sel == 0] == 7.0).all()


@pytest.mark.parametrize("H,P,d", [(2, 8, 72), (48, 32, 64), (1, 3, 128)])
def test_sig_drift_matches_oracle(H, P, d):
    import torch

    import context_state_reuse_amd as lib
    from oracle.planner import rel_drift
    rng = np.random.default_rng(H * 1000 + P)
    B = rng.normal(size=(H, P, P, d)).astype(np.float32)
    A = (B + rng.uniform(0, 0.3, size=(1, P, P, 1)) * rng.normal(size=B.shape)).astype(np.float32)
    B[:, 0, 1] = 0.0                                # ||B|| = 0: 0 if A is 0 too, else inf
    A[:, 0, 1] = 0.0
    B[:, 1, 0] = 0.0
    sel = (rng.uniform(size=(P, P)) < 0.6).astype(np.uint8)
    sel[0, 1] = sel[1, 0] = 1
    out = torch.full((P, P), -1.0, dtype=torch.float32, device="cuda")
    lib.ditango_sig_drift(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), sel, out)
    o = out.cpu().numpy()
    for q in range(P):
        for k in range(P):
            if not sel[q, k]:
                assert o[q, k] == -1.0
                continue
            ref = rel_drift(A[:, q, k], B[:, q, k])
            if math.isinf(ref):
                assert math.isinf(o[q, k])
            else:
                assert o[q, k] == pytest.approx(ref, rel=1e-5, abs=1e-7), (q, k)


def test_pair_stats_errors():
    import torch

    import context_state_reuse_amd as lib
    w = CASES[0]
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    LSE = torch.zeros((w.H, w.N), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.DitangoError) as e:          # nothing cached yet
        lib.ditango_pair_stats(cache, LSE, np.ones((w.P, w.P), np.uint8))
    assert e.value.code == lib.DITANGO_ENOCACHE


def test_planned_steps_match_oracle_with_their_masks():
    import torch

    import context_state_reuse_amd as lib
    w = _scaled("image", "image_plan", 1, 57, 97, 2, steps=8)
    g = 2
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    runner = lib.PlannedSteps(cache, lib.Planner(w.P, g, w.H, target_reuse=0.6, drift_max=0.1))
    stream = synth.InputStream(w)
    masks, outs, anchors = {}, {}, []
    for t in range(w.steps):
        qb, kb, vb = stream.next()
        mask, anchor, O, LSE = runner.step(t, to_device(qb), to_device(kb), to_device(vb))
        torch.cuda.synchronize()
        masks[t], outs[t] = mask.copy(), (O.cpu().numpy(), LSE.cpu().numpy())
        anchors.append(anchor)
        log(f"  [plan] step {t}: anchor {anchor}, fresh {int(mask.sum())}/{w.P * w.P}, eps {runner.planner.eps:.3g}")
        assert (np.diag(mask) == 1).all()
        for q in range(w.P):
            for j in range(-(-w.P // g)):
                mem = group_members(w.P, g, q, j)
                if mem:
                    assert len({int(mask[q, k]) for k in mem}) == 1, f"step {t}: group {j} of q={q} split"
    # warm-up anchors, selective steps, and (local drift ~0.015 per step) one drift anchor
    assert anchors[0] and anchors[1]
    assert not all(anchors), "no selective step in the run"
    assert any(anchors[2:]), "the local drift never triggered an anchor"
    # the oracle with the same masks
    orc = StateReuseOracle(w.N, w.P, w.d)
    stream = synth.InputStream(w)
    for t in range(w.steps):
        qb, kb, vb = stream.next()
        res = orc.step(t, masks[t], {h: (synth.bf16_bits_to_f64(qb[h]), synth.bf16_bits_to_f64(kb[h]),
                                         synth.bf16_bits_to_f64(vb[h])) for h in range(w.H)})
        for h in range(w.H):
            err = np.abs(outs[t][0][h].astype(np.float64) - res["O"][h])
            lerr = np.abs(outs[t][1][h].astype(np.float64) - res["LSE"][h])
            assert err.max() <= TOL_O_MAX and err.mean() <= TOL_O_MEAN and lerr.max() <= TOL_LSE, \
                f"step {t} head {h}: OUT {err.max():.3g}/{err.mean():.3g}, LSE {lerr.max():.3g}"
    assert math.isfinite(runner.planner.eps)


def test_planned_full_size_image_on_sampled_rows():
    """The full image workload (16 heads, 16384 tokens) for 8 planned steps;
    the oracle replays the chosen masks for two heads on sampled rows."""
    import torch

    import context_state_reuse_amd as lib
    from oracle.reuse import run_workload
    w = synth.get("image").scaled(steps=8)
    heads = [0, w.H - 1]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[q * w.S, min((q + 1) * w.S, w.N) - 1, *rng.integers(q * w.S, min((q + 1) * w.S, w.N), 4)]
                                     for q in range(w.P)]))
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    runner = lib.PlannedSteps(cache, lib.Planner(w.P, 2, w.H, target_reuse=0.75, drift_max=0.1))
    stream = synth.InputStream(w)
    masks, outs, anchors = {}, {}, []
    r_t = torch.tensor(rows, device="cuda")
    for t in range(w.steps):
        qb, kb, vb = stream.next()
        mask, anchor, O, LSE = runner.step(t, to_device(qb), to_device(kb), to_device(vb))
        masks[t] = mask.copy()
        outs[t] = (O[heads][:, r_t].cpu().numpy(), LSE[heads][:, r_t].cpu().numpy())
        anchors.append(anchor)
        log(f"  [plan image] step {t}: anchor {anchor}, fresh {int(mask.sum())}/{w.P * w.P}")
        del qb, kb, vb
    assert anchors[0] and anchors[1] and not all(anchors)
    ref = {}
    run_workload(w, heads=heads, rows=rows, masks=masks, on_step=lambda t, m, r: ref.__setitem__(t, r))
    for t in range(w.steps):
        for hi, h in enumerate(heads):
            err = np.abs(outs[t][0][hi].astype(np.float64) - ref[t]["O"][h])
            lerr = np.abs(outs[t][1][hi].astype(np.float64) - ref[t]["LSE"][h])
            assert err.max() <= TOL_O_MAX and err.mean() <= TOL_O_MEAN and lerr.max() <= TOL_LSE, \
                f"step {t} head {h}: OUT {err.max():.3g}/{err.mean():.3g}, LSE {lerr.max():.3g}"


def test_planned_steps_on_a_side_stream_match_the_current_stream():
    """The same planned steps driven on a second (default-priority) stream:
    every launch and every table copy of a step runs on that stream, so
    masks and outputs are bit-identical to the run on the current stream
    (all kernels here sum in a fixed order).  The statistics calls that
    allocate their outputs are run on the side stream too."""
    import torch

    import context_state_reuse_amd as lib
    w = _scaled("image", "image_plan_stream", 1, 57, 97, 2, steps=6)
    side = torch.cuda.Stream()
    runs = []
    for stream in (None, side):
        cache = lib.StateCache(w.H, w.N, w.d, w.P)
        runner = lib.PlannedSteps(cache, lib.Planner(w.P, 2, w.H, target_reuse=0.6, drift_max=0.1))
        inputs = synth.InputStream(w)
        got = []
        for t in range(w.steps):
            qb, kb, vb = inputs.next()
            Q, K, V = to_device(qb), to_device(kb), to_device(vb)
            if stream is not None:
                stream.wait_stream(torch.cuda.current_stream())    # inputs written on the current stream
            mask, anchor, O, LSE = runner.step(t, Q, K, V, stream)
            torch.cuda.synchronize()
            got.append((mask.copy(), anchor, O.cpu().numpy().copy(), LSE.cpu().numpy().copy()))
        if stream is not None:
            _, sig = lib.ditango_pair_stats(cache, None, np.eye(w.P, dtype=np.uint8), stream=stream, want_w=False)
            dr = lib.ditango_sig_drift(sig, sig, np.ones((w.P, w.P), np.uint8), stream=stream)
            torch.cuda.synchronize()
            assert (dr.cpu().numpy() == 0).all()
        runs.append(got)
        log(f"  [stream] run on {'side' if stream is not None else 'current'} stream: "
            f"anchors {[t for t, g in enumerate(got) if g[1]]}")
    for t, (a, b) in enumerate(zip(*runs)):
        assert (a[0] == b[0]).all() and a[1] == b[1], f"step {t}: masks differ"
        assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3]), f"step {t}: outputs differ"


def test_oracle_planner_on_oracle_statistics_picks_the_same_masks():
    """End to end: the library's planner, fed the GPU's fp32 statistics,
    against the oracle planner fed the oracle's own fp64 statistics (local
    signatures of the step's fresh local states, importance from the merged
    LSE, signatures of every pair before and after an anchor step), step by
    step on the same inputs.  Every decision must agree -- the anchor flag,
    and per (query partition, group) compute or reuse -- except a decision
    within MARGIN (relative) of its threshold: a predicted group error within
    MARGIN of eps, or the largest local drift within MARGIN of the anchor
    bound, which fp32 statistics may flip legitimately (right after an
    anchor the group whose error sets eps sits on it by construction).  The
    oracle then follows the library's mask, so both runs keep the same
    cache.  The exempt decisions are counted and bounded."""
    import torch

    import context_state_reuse_amd as lib
    from oracle.planner import AnchorPlanner
    from oracle.state import partial_state, partition_bounds
    from synth import bf16_bits_to_f64

    MARGIN = 0.05
    w = _scaled("image", "image_plan_e2e", 1, 57, 97, 2, steps=12)
    g, rho, dmax = 2, 0.6, 0.1
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    runner = lib.PlannedSteps(cache, lib.Planner(w.P, g, w.H, target_reuse=rho, drift_max=dmax))
    orc = StateReuseOracle(w.N, w.P, w.d)
    opl = AnchorPlanner(w.P, g, rho, dmax)
    bounds = partition_bounds(w.N, w.P)
    stream = synth.InputStream(w)

    def cache_sigs():
        sig = np.zeros((w.H, w.P, w.P, w.d))
        for (h, q, k), (o, _) in orc.cache.items():
            sig[h, q, k] = pair_signature(o)
        return sig

    compared, exempt, selective = 0, 0, 0
    for t in range(w.steps):
        qb, kb, vb = stream.next()
        mask_l, anchor_l, _, _ = runner.step(t, to_device(qb), to_device(kb), to_device(vb))
        torch.cuda.synchronize()
        x = {h: (bf16_bits_to_f64(qb[h]), bf16_bits_to_f64(kb[h]), bf16_bits_to_f64(vb[h])) for h in range(w.H)}
        sig_local = np.zeros((w.H, w.P, w.P, w.d))
        if opl.n_anchors:
            for h, (Qh, Kh, Vh) in x.items():
                for q, (lo, hi) in enumerate(bounds):
                    sig_local[h, q, q] = pair_signature(partial_state(Qh[lo:hi], Kh[lo:hi], Vh[lo:hi], orc.scale)[0])
        mask_o, anchor_o = opl.plan(t, sig_local)
        near_anchor = bool(opl.n_anchors and t >= opl.warmup
                           and abs(float(np.max(opl.D)) - dmax) <= MARGIN * dmax)
        if near_anchor:
            exempt += 1
        else:
            compared += 1
            assert anchor_o == anchor_l, f"step {t}: anchor {anchor_l} on the GPU, {anchor_o} in the oracle"
        n_exempt_groups = 0
        if not anchor_o and not anchor_l:
            ase = opl.predicted_errors()
            for q in range(w.P):
                for j in range(opl.m):
                    mem = group_members(w.P, g, q, j)
                    if not mem:
                        continue
                    if abs(ase[q, j] - opl.eps) <= MARGIN * max(abs(opl.eps), 1e-12):
                        n_exempt_groups += 1
                        continue
                    compared += 1
                    assert mask_l[q, mem].tolist() == mask_o[q, mem].tolist(), \
                        f"step {t}: group {j} of query partition {q}: GPU {mask_l[q, mem]}, oracle {mask_o[q, mem]}"
            assert np.array_equal(np.diag(mask_l), np.ones(w.P, np.uint8))
        exempt += n_exempt_groups
        selective += not anchor_l
        opl.anchor = bool(anchor_l)
        mask = mask_l.copy()
        sig_old = cache_sigs() if opl.anchor and opl.n_anchors else None
        res = orc.step(t, mask, x)
        W = np.zeros((w.H, w.P, w.P))
        for h in range(w.H):
            lm = [res["LSE"][h][lo:hi] for lo, hi in bounds]
            W[h] = pair_weights([[orc.cache[(h, q, k)][1] for k in range(w.P)] for q in range(w.P)], lm)
        opl.update(t, mask, W, cache_sigs(), sig_old)
        log(f"  [{w.name}] step {t}: anchor {anchor_l}, fresh {int(mask_l.sum())}/{w.P * w.P}, "
            f"{n_exempt_groups} group decision(s) near eps{', anchor decision near the bound' if near_anchor else ''}")
    log(f"  [{w.name}] planner decisions: {compared} compared and equal, {exempt} near a threshold; "
        f"{selective} selective steps")
    assert selective >= 3, "the run must exercise selective steps"
    assert exempt * 5 <= compared + exempt, f"{exempt} of {compared + exempt} decisions near a threshold"
