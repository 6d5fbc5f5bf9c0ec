"""GPU parity of the grouped, composed state cache against the fp64 oracle
(oracle.groups), through the C ABI.

Same bar as the per-pair path: OUT max-abs <= 2e-2, mean-abs <= 2e-3, LSE
abs <= 1e-3 for every computed slot state and every merged output; the slot
decisions and t_c bit-exact; reused slots bit-identical to what was written
at their t_c.  Group merges (Dynamic Group State Compose) are checked the
same way on the steps after them.  Group sizes cover groups that lose q at
either end or in the middle (a gap in the key range) and an empty slot.
"""
import numpy as np
import pytest

import synth
from oracle.groups import GroupedStateReuseOracle, slot_members
from oracle.masks import all_fresh, all_reuse, step_mask

from gpu_run import log, run_group_steps
from test_gpu_parity import _sample_rows, _scaled, check_state

pytestmark = pytest.mark.gpu


def _oracle_steps(w, g, masks, steps, compose_at, rows=None, heads=None, budget_at=None):
    from synth import InputStream, bf16_bits_to_f64
    from oracle.groups import slot_bytes
    heads = list(range(w.H)) if heads is None else heads
    orc = GroupedStateReuseOracle(w.N, w.P, w.d, g, rows=rows)
    stream = InputStream(w, heads)
    out = {}
    for t in range(steps):
        qb, kb, vb = stream.next()
        if compose_at and t in compose_at:
            orc.compose_groups(compose_at[t])
        if budget_at and t in budget_at:
            orc.fit_memory(budget_at[t], 2, slot_bytes(w.H, w.N, w.P, w.d))
        m = masks[t] if masks and t in masks else step_mask(w, t)
        x = {h: (bf16_bits_to_f64(qb[i]), bf16_bits_to_f64(kb[i]), bf16_bits_to_f64(vb[i]))
             for i, h in enumerate(heads)}
        out[t] = (m.copy(), orc.step(t, m, x), orc.g)
    return out, orc


def _compare(w, g, masks=None, steps=None, compose_at=None, rows=None, heads=None, label=None, budget_at=None,
             state_dtype="fp32"):
    steps = w.steps if steps is None else steps
    ref, orc = _oracle_steps(w, g, masks, steps, compose_at, rows, heads, budget_at)
    heads = list(range(w.H)) if heads is None else heads
    rows_all = orc.rows
    import torch
    hsel = torch.tensor(heads, device="cuda")
    snap = {}
    worst = [0.0, 0.0, 0.0]

    def check(t, mask, computed, cache, O, LSE):
        omask, res, og = ref[t]
        assert np.array_equal(mask, omask), f"step {t}: mask differs"
        assert cache.g == og
        assert np.array_equal(computed, res["computed"]), f"step {t}: slot decisions differ"
        assert np.array_equal(cache.tc_matrix, res["tc"]), f"step {t}: t_c differs"
        ns = cache.n_slots
        assert len(cache.O) == ns
        for s in range(ns):
            Os, Ls = cache.O[s][hsel].float().cpu().numpy(), cache.LSE[s][hsel].cpu().numpy()
            for hi, h in enumerate(heads):
                for q in range(w.P):
                    if not slot_members(w.P, cache.g, q, s):
                        continue
                    r = orc.part_rows[q] - q * w.S
                    if r.size == 0:
                        continue
                    o, l = Os[hi, q, r], Ls[hi, q, r]
                    if computed[q, s]:
                        o_ref, l_ref = res["fresh"][(h, q, s)]
                        e = check_state(o, l, o_ref, l_ref, f"{label} step {t} head {h} slot ({q},{s})")
                        worst[:] = [max(a, b) for a, b in zip(worst, e)]
                    elif (t - 1) in ref and ref[t - 1][2] == og:
                        po, pl = snap[(h, q, s)]
                        assert np.array_equal(o, po) and np.array_equal(l, pl), f"step {t}: reused slot changed"
                    snap[(h, q, s)] = (o.copy(), l.copy())
        Oc, Lc = O[hsel].cpu().numpy(), LSE[hsel].cpu().numpy()
        for hi, h in enumerate(heads):
            check_state(Oc[hi, rows_all], Lc[hi, rows_all], res["O"][h], res["LSE"][h],
                        f"{label} step {t} head {h} merged")

    for fused in (False, True):       # two launches per step, then the fused group step launch
        snap.clear()
        run_group_steps(w, g, masks=masks, steps=steps, compose_at=compose_at, on_step=check, label=label,
                        budget_at=budget_at, fused=fused, state_dtype=state_dtype)
    log(f"  {label} ({state_dtype} states): worst slot state OUT max {worst[0]:.2e}, mean {worst[1]:.2e}, LSE {worst[2]:.2e}")


GROUPED = [
    (synth.get("tiny"), 2),                                              # groups of 2, P=4
    (_scaled("image", "image_small", 1, 57, 97, 2), 3),                  # d=72, P=8: q inside its group
    (_scaled("video_25", "video25_small", 5, 21, 29, 2), 4),             # d=128, P=8
    (_scaled("long", "long_small", 7, 19, 23, 2), 4),                    # P=16, ragged last partition
    (_scaled("stress", "stress_small", 5, 16, 27, 2), 4),                # d=64, P=32, S=68
    (_scaled("stress", "stress_g3", 5, 16, 27, 1, steps=4), 3),          # last group {30, 31}, gaps
    (_scaled("stress", "stress_g1", 3, 14, 19, 1, steps=3, P=31), 1),    # g = 1: 32 slots
]


@pytest.mark.parametrize("w,g", GROUPED, ids=[f"{w.name}_g{g}" for w, g in GROUPED])
def test_grouped_workload_matches_oracle(w, g):
    _compare(w, g, label=f"{w.name} g={g}")


GROUPED_BF16 = [GROUPED[1], GROUPED[3], GROUPED[4]]


@pytest.mark.parametrize("w,g", GROUPED_BF16, ids=[f"{w.name}_g{g}" for w, g in GROUPED_BF16])
def test_grouped_bf16_states_match_oracle(w, g):
    _compare(w, g, label=f"{w.name} g={g}", state_dtype="bf16")


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
def test_group_merges_match_oracle(state_dtype):
    """g = 1 -> 2 -> 4 with reuse across the merges, then fresh work at g = 4
    (group merges write the merged slot in the cache's own format)."""
    w = synth.get("video_100").scaled(name="merge_p8", F=3, Hh=13, W=21, H=2, P=8, steps=6)
    rng = np.random.default_rng(11)
    masks = {0: all_fresh(8), 1: (rng.random((8, 8)) < 0.4).astype(np.uint8), 2: all_reuse(8),
             3: all_reuse(8), 4: (rng.random((8, 8)) < 0.3).astype(np.uint8), 5: all_reuse(8)}
    _compare(w, 1, masks=masks, compose_at={2: 2, 4: 2}, label="merges", state_dtype=state_dtype)


def test_memory_budget_merges_match_oracle():
    """The memory trigger: a budget that lets the cache start at g = 1 (9
    slots), then one that forces a merge to g = 2 (5 slots), then one that
    forces two more (g = 8, 2 slots), with reuse across the merges."""
    from oracle.groups import slot_bytes
    w = synth.get("video_100").scaled(name="budget_p8", F=3, Hh=13, W=21, H=2, P=8, steps=6)
    sb = slot_bytes(w.H, w.N, w.P, w.d)       # fp32 slots, the cache's default
    rng = np.random.default_rng(5)
    masks = {0: all_fresh(8), 1: (rng.random((8, 8)) < 0.4).astype(np.uint8), 2: all_reuse(8),
             3: (rng.random((8, 8)) < 0.3).astype(np.uint8), 4: all_reuse(8), 5: all_reuse(8)}
    _compare(w, 1, masks=masks, budget_at={0: 9 * sb, 2: 5 * sb, 4: 2 * sb}, label="budget")


def test_group_aligned_masks_match_oracle():
    """Masks that select whole groups (local pair plus the nearest groups)."""
    from oracle.groups import nearest_groups_mask
    w = _scaled("stress", "stress_gmask", 5, 16, 27, 2, steps=4)
    m = nearest_groups_mask(w.P, 4, 2)
    _compare(w, 4, masks={0: all_fresh(w.P), 1: m, 2: m, 3: m}, compose_at={3: 2}, label="group masks")


def test_group_merge_frees_slots_and_reset():
    import torch
    import context_state_reuse_amd as lib
    w = synth.get("stress").scaled(name="free", F=2, Hh=16, W=27, H=2, steps=3)
    cache = lib.GroupedStateCache(w.H, w.N, w.d, w.P, 2)
    assert cache.n_slots == 17 and len(cache.O) == 17 and cache.O[0].dtype == torch.float32
    before = cache.device_bytes
    q = torch.zeros((w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    lib.ditango_group_attn_partial(q, q, q, all_fresh(w.P), cache)
    lib.ditango_group_cache_update(cache, all_fresh(w.P), 0)
    cache.compose(4)
    assert cache.g == 8 and cache.n_slots == 5 and len(cache.O) == 5
    assert cache.device_bytes * 17 == before * 5
    O, L = lib.ditango_group_merge(cache)
    torch.cuda.synchronize()
    # zero inputs: uniform attention, OUT = 0, LSE = log N
    assert float(O.abs().max()) == 0.0
    assert abs(float(L.mean()) - np.log(w.N)) < 1e-4
    cache.reset()
    assert cache.g == 2 and len(cache.O) == 17 and np.all(cache.tc == -1)
    with pytest.raises(lib.DitangoError):
        lib.ditango_group_merge(cache)


FULL_GROUPED = [("stress", 4, "fp32"), ("long", 4, "fp32"), ("video_25", 2, "fp32"), ("image", 3, "fp32"),
                ("stress", 4, "bf16")]


@pytest.mark.parametrize("name,g,state_dtype", FULL_GROUPED, ids=[f"{n}_g{g}_{sd}" for n, g, sd in FULL_GROUPED])
def test_full_size_grouped_sampled_rows(name, g, state_dtype):
    import torch
    w = synth.get(name)
    steps = min(w.steps, 3)
    _compare(w, g, steps=steps, rows=_sample_rows(w), heads=[0, w.H - 1], label=f"{name} g={g} full",
             state_dtype=state_dtype)
    torch.cuda.empty_cache()
