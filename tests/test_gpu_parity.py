"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar (bf16 inputs, fp32 accumulation): OUT max-abs <= 2e-2 and mean-abs
<= 2e-3, LSE abs <= 1e-3, for every fresh pair state and every merged
output; the selection mask, the reused set and t_c bit-exact; reused cache
slots bit-identical to what was written at their t_c.

The reduced and edge workloads run twice: partial, t_c update and merge as
three calls, and each step as one fused launch (ditango_step).

Reduced workloads keep each workload's d, P, mask policy and value recipe at
sizes the oracle finishes in seconds, with several key tiles, both query-tile
widths and ragged last partitions; the full-size workloads run through the
fused step launch (the benchmark's configuration) and are checked on sampled
rows (first, last and interior rows of every partition) of two heads.
"""
import numpy as np
import pytest

import synth
from oracle.masks import step_mask as oracle_mask
from oracle.reuse import run_workload

from gpu_run import log, run_steps

pytestmark = pytest.mark.gpu

TOL_O_MAX, TOL_O_MEAN, TOL_LSE = 2e-2, 2e-3, 1e-3


def check_state(o, l, o_ref, l_ref, what):
    err = np.abs(np.asarray(o, np.float64) - o_ref)
    lerr = np.abs(np.asarray(l, np.float64) - l_ref)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    assert err.max() <= TOL_O_MAX, f"{what}: OUT max-abs {err.max():.3g}"
    assert err.mean() <= TOL_O_MEAN, f"{what}: OUT mean-abs {err.mean():.3g}"
    assert lerr.max() <= TOL_LSE, f"{what}: LSE abs {lerr.max():.3g}"
    return err.max(), err.mean(), lerr.max()


def _scaled(base, name, F, Hh, W, H, **kw):
    return synth.get(base).scaled(name=name, F=F, Hh=Hh, W=W, H=H, **kw)


REDUCED = [
    synth.get("tiny"),                                           # full size: S=256, 256-row tiles
    _scaled("image", "image_small", 1, 57, 97, 2),               # d=72, S=692 (last 685)
    _scaled("video_100", "video100_small", 5, 21, 29, 2),        # d=128, S=381 (last 378)
    _scaled("video_50", "video50_small", 5, 21, 29, 2),
    _scaled("video_25", "video25_small", 5, 21, 29, 2),
    _scaled("long", "long_small", 7, 19, 23, 2),                 # d=128, P=16, S=192 (last 179)
    _scaled("stress", "stress_small", 5, 16, 27, 3),             # d=64, P=32, S=68 (last 52)
    _scaled("stress", "stress_tiny_parts", 3, 14, 19, 1, steps=4),  # S=25 (last 23)
]


def _run_full_compare(w, masks=None, label=None, state_dtype="fp32"):
    """Whole-tensor comparison of every step of a small workload."""
    ref = {}

    def keep(t, mask, res):
        ref[t] = (mask.copy(), res)

    run_workload(w, masks=masks, on_step=keep)
    snap = {}
    worst = [0, 0, 0]

    def check(t, mask, reused, cache, O, LSE):
        omask, res = ref[t]
        assert np.array_equal(mask, omask), f"step {t}: mask differs from the oracle's"
        assert np.array_equal(reused, res["reused"]), f"step {t}: reused set differs"
        assert np.array_equal(cache.tc_matrix, res["tc"]), f"step {t}: t_c differs"
        Oc, Lc = cache.O.float().cpu().numpy(), cache.LSE.cpu().numpy()
        P, S = w.P, w.S
        for h in range(w.H):
            for q in range(P):
                n = min(S, w.N - q * S)
                for k in range(P):
                    slot = q * P + k
                    if mask[q, k]:
                        o_ref, l_ref = res["fresh"][(h, q, k)]
                        e = check_state(Oc[h, slot, :n], Lc[h, slot, :n], o_ref, l_ref,
                                        f"{w.name} step {t} head {h} pair ({q},{k})")
                        worst[:] = [max(a, b) for a, b in zip(worst, e)]
                    else:
                        po, pl = snap[(h, slot)]
                        assert np.array_equal(Oc[h, slot, :n], po) and np.array_equal(Lc[h, slot, :n], pl), \
                            f"step {t}: reused slot {(h, q, k)} changed"
                    snap[(h, slot)] = (Oc[h, slot, :n].copy(), Lc[h, slot, :n].copy())
            check_state(O[h].cpu().numpy(), LSE[h].cpu().numpy(), res["O"][h], res["LSE"][h],
                        f"{w.name} step {t} head {h} merged")

    for fused in (False, True):       # three calls per step, then the fused step launch
        snap.clear()
        run_steps(w, masks=masks, on_step=check, label=label, fused=fused, state_dtype=state_dtype)
    log(f"  {label or w.name} ({state_dtype} states): worst pair state OUT max {worst[0]:.2e}, mean {worst[1]:.2e}, LSE {worst[2]:.2e}")


@pytest.mark.parametrize("w", REDUCED, ids=[w.name for w in REDUCED])
def test_reduced_workload_matches_oracle(w):
    _run_full_compare(w)


BF16_STATES = [REDUCED[0], REDUCED[1], REDUCED[4], REDUCED[5], REDUCED[6]]


@pytest.mark.parametrize("w", BF16_STATES, ids=[w.name for w in BF16_STATES])
def test_reduced_workload_bf16_states_match_oracle(w):
    """The opt-in bf16 state format (d = 64, 72, 128; P = 4 to 32) to the
    same bar: rounding a state's OUT to bf16 adds at most 2^-9 relative."""
    _run_full_compare(w, state_dtype="bf16")


EDGE = [
    ("single_partition", synth.get("video_100").scaled(name="p1", F=1, Hh=10, W=30, H=2, P=1, steps=2,
                                                      n_fresh=1)),
    ("one_token_partitions", synth.get("stress").scaled(name="s1", F=1, Hh=2, W=4, H=2, P=8, steps=3,
                                                         n_fresh=3)),
    ("one_token_last", synth.get("image").scaled(name="last1", F=1, Hh=1, W=13, H=1, P=4, steps=3)),
    ("many_heads_d72", synth.get("image").scaled(name="h9", F=1, Hh=10, W=20, H=9, P=3, steps=3)),
    ("radius2_d128", synth.get("tiny").scaled(name="r2", F=1, Hh=17, W=31, H=2, d=128, P=6, steps=3,
                                              n_fresh=2)),
]


@pytest.mark.parametrize("w", [e[1] for e in EDGE], ids=[e[0] for e in EDGE])
def test_edge_shapes_match_oracle(w):
    _run_full_compare(w)


def test_random_masks_each_step():
    """Per-step random masks with very different fresh fractions (cache churn)."""
    w = synth.get("video_100").scaled(name="churn", F=2, Hh=11, W=23, H=2, P=5, steps=6)
    rng = np.random.default_rng(7)
    masks = {t: (rng.random((5, 5)) < f).astype(np.uint8) for t, f in zip(range(1, 6), (0.1, 0.9, 0.0, 0.5, 0.3))}
    _run_full_compare(w, masks=masks, label="churn")


def test_tiny_fp32_masters_error():
    """The tiny workload is specified in fp32; the library computes on bf16
    copies of the inputs.  Error of the GPU output against the fp64 oracle
    run on the unrounded fp32 masters, reported and bounded to first order:
    rounding q and k to bf16 (relative error <= 2^-9 each) moves a score by
    at most B = scale * 2^-8 * max_ij sum_c |q_ic k_jc|, so the LSE by at most
    B and OUT by at most (2B + 2^-9) max|v|, on top of the bf16 parity bars."""
    from synth import InputStream
    w = synth.get("tiny")
    scale = 1.0 / np.sqrt(w.d)
    B, vmax = 0.0, 0.0
    stream = InputStream(w)
    for t in range(w.steps):
        stream.advance()
        q, k, v = (m.astype(np.float64) for m in stream.masters)
        for h in range(w.H):
            B = max(B, scale * 2.0 ** -8 * (np.abs(q[h]) @ np.abs(k[h]).T).max())
            vmax = max(vmax, np.abs(v[h]).max())
    ref = {}
    run_workload(w, fp32_masters=True, on_step=lambda t, m, r: ref.__setitem__(t, r))
    worst = [0.0, 0.0, 0.0]

    def check(t, mask, reused, cache, O, LSE):
        for h in range(w.H):
            e = np.abs(O[h].cpu().numpy().astype(np.float64) - ref[t]["O"][h])
            le = np.abs(LSE[h].cpu().numpy().astype(np.float64) - ref[t]["LSE"][h])
            worst[:] = [max(worst[0], e.max()), max(worst[1], e.mean()), max(worst[2], le.max())]

    run_steps(w, on_step=check, fused=True)
    log(f"  tiny on fp32 masters: merged OUT max {worst[0]:.2e} mean {worst[1]:.2e}, LSE max {worst[2]:.2e} "
        f"(first-order bounds: LSE {B + TOL_LSE:.2e}, OUT {(2 * B + 2.0 ** -9) * vmax + TOL_O_MAX:.2e})")
    assert worst[2] <= B + TOL_LSE
    assert worst[0] <= (2 * B + 2.0 ** -9) * vmax + TOL_O_MAX


# ---------------------------------------------------------------- full size

def _sample_rows(w, per_part=4, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for q in range(w.P):
        lo, hi = q * w.S, min((q + 1) * w.S, w.N)
        rows += [lo, hi - 1] + list(rng.integers(lo, hi, per_part - 2))
    return np.unique(np.array(rows))


FULL = [(n, "fp32") for n in ("image", "video_100", "video_50", "video_25", "long", "stress")] + \
       [("long", "bf16"), ("stress", "bf16")]


@pytest.mark.parametrize("name,state_dtype", FULL, ids=[f"{n}_{s}" for n, s in FULL])
def test_full_size_sampled_rows(name, state_dtype):
    import torch
    w = synth.get(name)
    heads = [0, w.H - 1]
    rows = _sample_rows(w)
    P, S = w.P, w.S
    qidx = rows // S
    ridx = rows - qidx * S
    got = {}

    def grab(t, mask, reused, cache, O, LSE):
        h_t = torch.tensor(heads, device="cuda")
        r_t = torch.tensor(rows, device="cuda")
        slots = torch.tensor(qidx[:, None] * P + np.arange(P)[None, :], device="cuda")  # [rows, P]
        i_t = torch.tensor(ridx, device="cuda")
        so = cache.O[h_t[:, None, None], slots[None], i_t[None, :, None]].float().cpu().numpy()   # [2, rows, P, d]
        sl = cache.LSE[h_t[:, None, None], slots[None], i_t[None, :, None]].cpu().numpy()
        got[t] = dict(mask=mask.copy(), reused=reused.copy(), tc=cache.tc_matrix,
                      O=O[h_t][:, r_t].cpu().numpy(), LSE=LSE[h_t][:, r_t].cpu().numpy(), so=so, sl=sl)

    run_steps(w, on_step=grab, fused=True, state_dtype=state_dtype)   # the launch bench.py times
    prev = None
    worst = [0, 0, 0]
    ref_steps = {}
    run_workload(w, heads=heads, rows=rows, on_step=lambda t, m, r: ref_steps.__setitem__(t, (m.copy(), r)))
    for t in range(w.steps):
        m, res = ref_steps[t]
        g = got[t]
        assert np.array_equal(g["mask"], m) and np.array_equal(g["mask"], oracle_mask(w, t))
        assert np.array_equal(g["reused"], res["reused"]) and np.array_equal(g["tc"], res["tc"])
        for hi, h in enumerate(heads):
            e = check_state(g["O"][hi], g["LSE"][hi], res["O"][h], res["LSE"][h], f"{name} step {t} head {h} merged")
            worst[:] = [max(a, b) for a, b in zip(worst, e)]
            for q in range(P):
                sel = np.flatnonzero(qidx == q)
                for k in range(P):
                    if m[q, k]:
                        o_ref, l_ref = res["fresh"][(h, q, k)]
                        check_state(g["so"][hi, sel, k], g["sl"][hi, sel, k], o_ref, l_ref,
                                    f"{name} step {t} head {h} pair ({q},{k})")
                    elif prev is not None:
                        assert np.array_equal(g["so"][hi, sel, k], prev["so"][hi, sel, k])
                        assert np.array_equal(g["sl"][hi, sel, k], prev["sl"][hi, sel, k])
        prev = g
    log(f"  {name} ({state_dtype} states): sampled merged OUT max {worst[0]:.2e} mean {worst[1]:.2e} LSE {worst[2]:.2e}")


# ---------------------------------------------------------------- reuse laws

SMALL = _scaled("video_50", "laws", 3, 12, 19, 2)


def test_all_reuse_step_reproduces_cached_output_bitwise():
    outs = {}
    masks = {1: np.zeros((SMALL.P, SMALL.P), np.uint8)}
    run_steps(SMALL, masks=masks, steps=2,
              on_step=lambda t, m, r, c, O, L: outs.__setitem__(t, (O.cpu().numpy(), L.cpu().numpy())))
    assert np.array_equal(outs[1][0], outs[0][0]) and np.array_equal(outs[1][1], outs[0][1])


def test_zero_drift_any_mask_equals_all_fresh_bitwise():
    w = SMALL.scaled(sigma=0.0, steps=4)
    ref = {}
    run_steps(w, masks={t: np.ones((w.P, w.P), np.uint8) for t in range(4)}, steps=1,
              on_step=lambda t, m, r, c, O, L: ref.__setitem__(0, (O.cpu().numpy(), L.cpu().numpy())))
    rng = np.random.default_rng(3)
    masks = {t: (rng.random((w.P, w.P)) < 0.3).astype(np.uint8) for t in range(1, 4)}

    def check(t, m, r, c, O, L):
        assert np.array_equal(O.cpu().numpy(), ref[0][0]) and np.array_equal(L.cpu().numpy(), ref[0][1]), t

    run_steps(w, masks=masks, on_step=check)


def test_deterministic_across_runs():
    outs = []
    for _ in range(2):
        res = {}
        run_steps(SMALL, steps=3, on_step=lambda t, m, r, c, O, L: res.__setitem__(t, (O.cpu().numpy(), L.cpu().numpy())))
        outs.append(res)
    for t in range(3):
        assert np.array_equal(outs[0][t][0], outs[1][t][0]) and np.array_equal(outs[0][t][1], outs[1][t][1])


def test_merge_invariant_to_slot_order():
    """Composition is commutative: permuting the KV slots of each query
    partition changes the merged output only by fp32 rounding."""
    import torch

    import context_state_reuse_amd as lib
    w = SMALL
    base = {}

    def perm(t, m, r, cache, O, L):
        base["O"], base["L"] = O.clone(), L.clone()
        P = w.P
        rng = np.random.default_rng(11)
        idx = np.concatenate([q * P + rng.permutation(P) for q in range(P)])
        it = torch.tensor(idx, device="cuda")
        cache.O.copy_(cache.O[:, it].clone())
        cache.LSE.copy_(cache.LSE[:, it].clone())
        O2, L2 = lib.ditango_state_merge(cache)
        torch.cuda.synchronize()
        rel = ((O2 - base["O"]).abs().max() / base["O"].abs().max()).item()
        assert rel <= 1e-6, rel
        assert (L2 - base["L"]).abs().max().item() <= 1e-5

    run_steps(w, steps=1, on_step=perm)


def test_enocache_before_any_launch():
    import torch

    import context_state_reuse_amd as lib
    w = SMALL
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    x = torch.zeros((w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.DitangoError) as e:
        lib.ditango_attn_partial(x, x, x, lib.ditango_mask_build("nearest", w.P, 2), cache)
    assert e.value.code == lib.DITANGO_ENOCACHE
    with pytest.raises(lib.DitangoError) as e:
        lib.ditango_state_merge(cache)
    assert e.value.code == lib.DITANGO_ENOCACHE
