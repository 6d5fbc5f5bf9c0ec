"""GPU parity on seeded random shapes and masks (both caches) against the
fp64 oracles: head dims 64/72/128, 1 to 32 partitions, token counts that
leave ragged and one-token partitions, several heads, per-step random masks
including all-reuse steps; group sizes from 1 to P.  Both caches run as
separate launches with fp32 states and as fused launches, with fp32 states
in even-numbered cases and bf16 states in odd-numbered ones."""
import numpy as np
import pytest

import synth
from oracle.groups import GroupedStateReuseOracle, n_slots
from oracle.masks import all_fresh
from oracle.reuse import run_workload

from gpu_run import run_group_steps, run_steps
from test_gpu_parity import check_state

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 72, 128]))
        P = int(rng.integers(1, 33))
        while True:
            F, Hh, W = 1, int(rng.integers(1, 9)), int(rng.integers(P, 4 * P + 40))
            N = F * Hh * W
            S = -(-N // P)
            if N >= P and (P - 1) * S < N:
                break
        H = int(rng.integers(1, 4))
        steps = int(rng.integers(2, 5))
        w = synth.get("tiny").scaled(name=f"rand{i}", F=F, Hh=Hh, W=W, H=H, d=d, P=P, steps=steps,
                                     sigma=0.05)
        masks = {0: all_fresh(P)}
        for t in range(1, steps):
            m = (rng.random((P, P)) < rng.choice([0.0, 0.2, 0.6])).astype(np.uint8)
            m[np.arange(P), np.arange(P)] = 1 if rng.random() < 0.8 else m[np.arange(P), np.arange(P)]
            masks[t] = m
        g = int(rng.integers(1, P + 1)) if P > 1 else 1
        while n_slots(P, g) > 32:
            g += 1
        out.append((w, masks, g))
    return out


CASES = _cases()


@pytest.mark.parametrize("w,masks,g", CASES, ids=[f"{w.name}_d{w.d}_P{w.P}_N{w.N}_g{g}" for w, masks, g in CASES])
def test_random_shape_both_caches(w, masks, g):
    ref = {}
    run_workload(w, masks=masks, on_step=lambda t, m, r: ref.__setitem__(t, r))

    def check(t, mask, reused, cache, O, LSE):
        assert np.array_equal(cache.tc_matrix, ref[t]["tc"])
        for h in range(w.H):
            check_state(O[h].cpu().numpy(), LSE[h].cpu().numpy(), ref[t]["O"][h], ref[t]["LSE"][h],
                        f"{w.name} step {t} head {h}")

    fused_dtype = "bf16" if int(w.name[4:]) % 2 else "fp32"
    run_steps(w, masks=masks, on_step=check, label=w.name)
    run_steps(w, masks=masks, on_step=check, label=w.name, fused=True, state_dtype=fused_dtype)

    from synth import InputStream, bf16_bits_to_f64
    orc = GroupedStateReuseOracle(w.N, w.P, w.d, g)
    stream = InputStream(w)
    gref = {}
    for t in range(w.steps):
        qb, kb, vb = stream.next()
        x = {h: (bf16_bits_to_f64(qb[h]), bf16_bits_to_f64(kb[h]), bf16_bits_to_f64(vb[h])) for h in range(w.H)}
        gref[t] = orc.step(t, masks[t], x)

    def gcheck(t, mask, computed, cache, O, LSE):
        assert np.array_equal(computed, gref[t]["computed"]) and np.array_equal(cache.tc_matrix, gref[t]["tc"])
        for h in range(w.H):
            check_state(O[h].cpu().numpy(), LSE[h].cpu().numpy(), gref[t]["O"][h], gref[t]["LSE"][h],
                        f"{w.name} grouped g={g} step {t} head {h}")

    run_group_steps(w, g, masks=masks, on_step=gcheck, label=f"{w.name} g={g}")
    run_group_steps(w, g, masks=masks, on_step=gcheck, label=f"{w.name} g={g}", fused=True, state_dtype=fused_dtype)
    run_group_steps(w, g, masks=masks, on_step=gcheck, label=f"{w.name} g={g}", fused=True)
