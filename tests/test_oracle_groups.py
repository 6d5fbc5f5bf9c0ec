"""Pins of the grouped, composed state cache oracle (CPU only).

What fixes it independently of its own code: the Fig. 6 example (CP = 4,
rank 0: the remote partitions 2 and 3 composed and cached, 0 and 1 fresh);
with g = 1 it is the per-pair form, whose oracle is pinned on its own; with
every slot fresh it is full softmax attention; a fresh group state is the
attention state over the union of its members' keys (computed here in one
shot, not by composition); merging groups (Dynamic Group State Compose) does
not change what an all-reuse step returns (associativity of Eq. 4).
"""
import copy
import math
import os

import numpy as np
import pytest

import synth
from oracle.groups import (GroupedStateReuseOracle, group_decisions, n_slots,
                           nearest_groups_mask, slot_members)
from oracle.masks import all_fresh, all_reuse, radius_mask
from oracle.reuse import ReuseError, StateReuseOracle
from oracle.state import compose, compose2, partial_state, partition_bounds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SMALL = synth.get("tiny").scaled(name="tiny_small", F=2, Hh=6, W=7, H=2, d=8, P=4, steps=4)


def _inputs(w, t, heads=None):
    q, k, v = synth.step_inputs(w, t)
    heads = range(w.H) if heads is None else heads
    return {h: (synth.bf16_bits_to_f64(q[h]), synth.bf16_bits_to_f64(k[h]), synth.bf16_bits_to_f64(v[h]))
            for h in heads}


def _brute_state(q, k, v, scale):
    """Attention state by its definition, one softmax over all the keys given."""
    z = scale * (q @ k.T)
    lse = np.array([math.log(sum(math.exp(x) for x in row)) for row in z])
    out = np.exp(z - lse[:, None]) @ v
    return out, lse


def test_slot_layout_example():
    # P = 5, g = 2: groups {0,1} {2,3} {4}
    assert n_slots(5, 2) == 4 and n_slots(32, 4) == 9 and n_slots(16, 16) == 2
    assert slot_members(5, 2, 0, 0) == [0]
    assert slot_members(5, 2, 0, 1) == [1]          # the local group loses q
    assert slot_members(5, 2, 2, 1) == [0, 1]
    assert slot_members(5, 2, 2, 2) == [3]
    assert slot_members(5, 2, 4, 3) == []           # group {4} of query partition 4 is empty
    assert slot_members(6, 3, 4, 2) == [3, 5]       # q inside its group: members on both sides


def test_group_decisions_example():
    mask = np.array([[1, 0, 0, 1, 0],
                     [0, 1, 0, 0, 0],
                     [1, 0, 1, 1, 0],
                     [0, 0, 0, 0, 0],
                     [0, 0, 0, 0, 1]], dtype=np.uint8)
    expect = np.array([[1, 0, 1, 0],      # group {2,3} has a fresh member (3)
                       [1, 0, 0, 0],
                       [1, 1, 1, 0],      # {0,1}: 0 fresh; {3}: fresh
                       [0, 0, 0, 0],
                       [1, 0, 0, 0]],     # last slot of q=4 is empty, never computed
                      dtype=np.uint8)
    assert np.array_equal(group_decisions(mask, 2), expect)


def _fig6():
    rec = {}
    with open(os.path.join(GOLDEN, "fig6_cp4_rank0.txt")) as f:
        for ln in f:
            if ln.startswith("#") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            rec[k.strip()] = [int(x) for x in v.split()]
    return rec


def test_fig6_grouped_cache():
    """CP = 4, g = 2, rank 0: step t - 1 caches AS(2+3); step t computes
    AS(0), AS(1) fresh and composes them with the cached composite."""
    rec = _fig6()
    P, q = rec["P"][0], rec["query_partition"][0]
    w = SMALL
    assert w.P == P
    s = 1 / math.sqrt(w.d)
    b = partition_bounds(w.N, P)
    x0, x1 = _inputs(w, 0, [0])[0], _inputs(w, 1, [0])[0]
    lo, hi = b[q]
    st = lambda x, k: partial_state(x[0][lo:hi], x[1][b[k][0]:b[k][1]], x[2][b[k][0]:b[k][1]], s)
    cached = compose2(*[st(x0, k) for k in rec["reused"]])
    expect = compose([st(x1, k) for k in rec["fresh"]] + [cached])

    mask1 = radius_mask(P, 1)
    mask1[q] = 0
    mask1[q, rec["fresh"]] = 1
    orc = GroupedStateReuseOracle(w.N, P, w.d, g=2)
    orc.step(0, all_fresh(P), {0: x0})
    r = orc.step(1, mask1, {0: x1})
    np.testing.assert_allclose(r["O"][0][lo:hi], expect[0], atol=1e-13)
    np.testing.assert_allclose(r["LSE"][0][lo:hi], expect[1], atol=1e-13)
    assert list(r["computed"][q]) == [1, 1, 0]       # local, group {1}, group {2,3}
    assert list(r["tc"][q]) == [1, 1, 0]


def test_group_size_one_is_the_per_pair_form():
    w = SMALL
    P = w.P
    rng = np.random.default_rng(7)
    grp = GroupedStateReuseOracle(w.N, P, w.d, g=1)
    pair = StateReuseOracle(w.N, P, w.d)
    for t in range(4):
        m = all_fresh(P) if t == 0 else (rng.random((P, P)) < 0.45).astype(np.uint8)
        x = _inputs(w, t)
        rg, rp = grp.step(t, m, x), pair.step(t, m, x)
        for h in range(w.H):
            np.testing.assert_allclose(rg["O"][h], rp["O"][h], atol=1e-13, rtol=0)
            np.testing.assert_allclose(rg["LSE"][h], rp["LSE"][h], atol=1e-13, rtol=0)
        for q in range(P):
            assert rg["tc"][q, 0] == rp["tc"][q, q]
            for k in range(P):
                if k != q:
                    assert rg["tc"][q, 1 + k] == rp["tc"][q, k]


@pytest.mark.parametrize("g", [2, 3, 4, 5])
def test_all_fresh_is_full_attention(g):
    w = synth.get("tiny").scaled(name="tiny_ragged", F=1, Hh=1, W=37, H=1, d=8, P=5, steps=1)
    assert w.N % w.P != 0
    (Q, K, V), = _inputs(w, 0).values()
    r = GroupedStateReuseOracle(w.N, w.P, w.d, g=g).step(0, all_fresh(w.P), {0: (Q, K, V)})
    o, l = _brute_state(Q, K, V, 1 / math.sqrt(w.d))
    np.testing.assert_allclose(r["O"][0], o, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][0], l, atol=1e-12)


@pytest.mark.parametrize("q,s", [(4, 2), (3, 2), (5, 2), (0, 1), (2, 1)])
def test_fresh_group_state_is_attention_over_its_members(q, s):
    """P = 6, g = 3: groups {0,1,2} {3,4,5}; q = 4 leaves {3,5} (a gap)."""
    w = synth.get("tiny").scaled(name="tiny_g3", F=1, Hh=6, W=7, H=1, d=8, P=6, steps=1)
    (Q, K, V), = _inputs(w, 0).values()
    b = partition_bounds(w.N, w.P)
    orc = GroupedStateReuseOracle(w.N, w.P, w.d, g=3)
    r = orc.step(0, all_fresh(w.P), {0: (Q, K, V)})
    mem = slot_members(w.P, 3, q, s)
    keys = np.concatenate([np.arange(*b[k]) for k in mem])
    lo, hi = b[q]
    o, l = _brute_state(Q[lo:hi], K[keys], V[keys], 1 / math.sqrt(w.d))
    got = r["fresh"][(0, q, s)]
    np.testing.assert_allclose(got[0], o, atol=1e-13)
    np.testing.assert_allclose(got[1], l, atol=1e-13)


def test_merging_groups_keeps_the_reused_output():
    w = SMALL.scaled(name="small_p8", P=8)
    P = w.P
    orc = GroupedStateReuseOracle(w.N, P, w.d, g=1)
    orc.step(0, all_fresh(P), _inputs(w, 0))
    orc.step(1, radius_mask(P, 1), _inputs(w, 1))
    twin = copy.deepcopy(orc)
    ref = twin.step(2, all_reuse(P), _inputs(w, 2))
    tc_before = orc.tc.copy()
    orc.compose_groups(2)
    assert orc.g == 2 and orc.tc.shape == (P, n_slots(P, 2))
    # q = 3: new group 1 covers old groups 2, 3 = partitions {2, 3} minus {3}
    assert orc.tc[3, 2] == tc_before[3, 1 + 2]
    # q = 0: new group 1 = partitions {2, 3}: fresh at 1 for neither -> oldest is 0
    assert orc.tc[0, 2] == min(tc_before[0, 3], tc_before[0, 4]) == 0
    # q = 2: new group 0 = partitions {0, 1}: 0 last fresh at 0, 1 at 1 -> the oldest, 0
    assert (tc_before[2, 1], tc_before[2, 2]) == (0, 1) and orc.tc[2, 1] == 0
    # q = 5: new group 2 = {4, 5} minus 5 -> t_c of old group 4 (fresh at 1)
    assert orc.tc[5, 3] == tc_before[5, 1 + 4] == 1
    got = orc.step(2, all_reuse(P), _inputs(w, 2))
    for h in range(w.H):
        np.testing.assert_allclose(got["O"][h], ref["O"][h], atol=1e-13)
        np.testing.assert_allclose(got["LSE"][h], ref["LSE"][h], atol=1e-13)
    orc.compose_groups(2)
    assert orc.g == 4 and orc.tc.shape == (P, 3)
    got = orc.step(3, all_reuse(P), _inputs(w, 3))
    for h in range(w.H):
        np.testing.assert_allclose(got["O"][h], ref["O"][h], atol=1e-13)
    # a fresh step at the coarser size is full attention again
    x = _inputs(w, 3)
    got = orc.step(3, all_fresh(P), x)
    for h in range(w.H):
        o, l = _brute_state(*x[h], 1 / math.sqrt(w.d))
        np.testing.assert_allclose(got["O"][h], o, atol=1e-12)
        np.testing.assert_allclose(got["LSE"][h], l, atol=1e-12)


def test_reuse_without_state_and_reset():
    w = SMALL
    orc = GroupedStateReuseOracle(w.N, w.P, w.d, g=2)
    with pytest.raises(ReuseError):
        orc.step(0, all_reuse(w.P), _inputs(w, 0))
    with pytest.raises(ReuseError):
        orc.compose_groups(2)
    orc.step(0, all_fresh(w.P), _inputs(w, 0))
    orc.compose_groups(2)
    orc.reset()
    assert orc.g == 2 and np.all(orc.tc == -1) and orc.tc.shape == (w.P, n_slots(w.P, 2))


def test_nearest_groups_mask_example():
    """P = 8, g = 2 (groups {0,1} {2,3} {4,5} {6,7}), two nearest groups, by hand:
    q=0: {1} at 1, {2,3} at 2 -> 0,1,2,3;  q=3: {2} at 1, {4,5} at 1 -> 2,3,4,5;
    q=4: {2,3} at 1 (lower index wins the tie with {5}), {5} at 1 -> 2,3,4,5;
    q=7: {6} at 1, {4,5} at 2 -> 4,5,6,7."""
    m = nearest_groups_mask(8, 2, 2)
    assert list(np.flatnonzero(m[0])) == [0, 1, 2, 3]
    assert list(np.flatnonzero(m[3])) == [2, 3, 4, 5]
    assert list(np.flatnonzero(m[4])) == [2, 3, 4, 5]
    assert list(np.flatnonzero(m[7])) == [4, 5, 6, 7]
    # P = 5, g = 2, one group: q = 4 (its own group {4} is empty) takes {2, 3}
    m = nearest_groups_mask(5, 2, 1)
    assert list(np.flatnonzero(m[4])) == [2, 3, 4] and list(np.flatnonzero(m[0])) == [0, 1]
    assert np.array_equal(nearest_groups_mask(6, 3, 0), np.eye(6, dtype=np.uint8))
    # P = 8, g = 4, one group: for q = 4 both {0..3} and {5,6,7} are at distance 1
    # (their closest members 3 and 5); the lower group wins
    assert list(np.flatnonzero(nearest_groups_mask(8, 4, 1)[4])) == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("P,g,n", [(32, 4, 2), (16, 4, 1), (8, 2, 1), (13, 3, 2), (32, 8, 3), (7, 7, 1)])
def test_nearest_groups_mask_is_group_aligned(P, g, n):
    """Every group is wholly fresh or wholly reused, and each row keeps q plus
    the members of exactly min(n, non-empty groups) groups."""
    m = nearest_groups_mask(P, g, n)
    for q in range(P):
        assert m[q, q] == 1
        chosen = 0
        for s in range(1, n_slots(P, g)):
            mem = slot_members(P, g, q, s)
            vals = {int(m[q, k]) for k in mem}
            assert len(vals) <= 1
            chosen += vals == {1}
        live = sum(1 for s in range(1, n_slots(P, g)) if slot_members(P, g, q, s))
        assert chosen == min(n, live)


def test_memory_trigger_merge_counts():
    """Merges by k needed to fit a budget: the cache holds 1 + ceil(P / g)
    slots, so for P = 32 and g = 1, 2, 4, 8, 16, 32 it holds 33, 17, 9, 5,
    3, 2 slots (counted by hand)."""
    from oracle.groups import merges_to_fit, n_slots
    assert [n_slots(32, g) for g in (1, 2, 4, 8, 16, 32)] == [33, 17, 9, 5, 3, 2]
    B = 1000
    want = {33: 0, 32: 1, 17: 1, 16: 2, 9: 2, 8: 3, 5: 3, 4: 4, 3: 4, 2: 5}
    for slots, n in want.items():
        assert merges_to_fit(32, 1, 2, B, slots * B) == n, slots
    assert merges_to_fit(32, 1, 4, B, 9 * B) == 1          # g = 4 in one merge by 4
    assert merges_to_fit(32, 1, 4, B, 8 * B) == 2          # then g = 16: 3 slots
    assert merges_to_fit(8, 3, 2, B, 3 * B) == 1           # g = 3 -> 6: 1 + 2 slots
    with pytest.raises(ValueError):
        merges_to_fit(32, 1, 2, B, 2 * B - 1)              # not even one group fits
    from oracle.groups import slot_bytes
    assert slot_bytes(2, 10, 4, 64) == 4 * 2 * 4 * 3 * 65        # S = ceil(10 / 4) = 3; fp32 OUT and LSE
    assert slot_bytes(2, 10, 4, 64, out_bytes=2) == 2 * 4 * 3 * (2 * 64 + 4)   # bf16 OUT


def test_memory_trigger_merges_like_explicit_compose():
    """fit_memory performs exactly the merges it counts: the same cache as
    explicit compose_groups calls, and an all-reuse step after it returns
    the output of the step before (merging only recomposes cached states)."""
    from oracle.groups import GroupedStateReuseOracle, merges_to_fit
    from oracle.masks import all_fresh, all_reuse
    rng = np.random.default_rng(3)
    N, P, d = 60, 8, 8
    x = {0: tuple(rng.standard_normal((N, d)) for _ in range(3))}
    a = GroupedStateReuseOracle(N, P, d, 1)
    b = GroupedStateReuseOracle(N, P, d, 1)
    r0 = a.step(0, all_fresh(P), x)
    b.step(0, all_fresh(P), x)
    assert merges_to_fit(P, 1, 2, 10, 30) == 2              # 9 slots -> 5 -> 3
    assert a.fit_memory(30, 2, 10) == 2 and a.g == 4
    b.compose_groups(2)
    b.compose_groups(2)
    assert b.g == 4 and np.array_equal(a.tc, b.tc)
    for key in b.cache:
        assert np.array_equal(a.cache[key][0], b.cache[key][0])
    r1 = a.step(1, all_reuse(P), x)
    assert np.abs(r1["O"][0] - r0["O"][0]).max() < 1e-12
    assert a.fit_memory(30, 2, 10) == 0                     # already fits
