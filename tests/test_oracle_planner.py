"""Pins of the planner oracle (CPU only).

Fixed independently of its code:
* the importance of pair (q, k), the mean normalised weight of partition k
  over q's rows, is the share of q's softmax attention mass that falls on
  k's keys -- checked against full attention computed by brute force, and
  it sums to 1 over k;
* a pair's signature is the mean over q's rows of attention restricted to
  k's keys -- brute force as well;
* drift and the reuse threshold against closed forms;
* the planner against a scenario worked out by hand: anchors at warm-up and
  on drift, the scale ratios, eps from the corrected errors, the group
  decisions between anchors and the per-group compute records.
"""
import math

import numpy as np
import pytest

import synth
from oracle.planner import AnchorPlanner, group_members, pair_signature, pair_weights, rel_drift, reuse_threshold
from oracle.state import compose, partial_state, partition_bounds


def _head(w, t=0, h=0):
    q, k, v = synth.step_inputs(w, t)
    return synth.bf16_bits_to_f64(q[h]), synth.bf16_bits_to_f64(k[h]), synth.bf16_bits_to_f64(v[h])


RAGGED = synth.get("tiny").scaled(name="tiny_ragged_p", F=1, Hh=1, W=45, H=1, d=8, P=4, steps=2)


def _slot_states(w, Q, K, V):
    b = partition_bounds(w.N, w.P)
    s = 1 / math.sqrt(w.d)
    return b, [[partial_state(Q[lo:hi], K[klo:khi], V[klo:khi], s) for (klo, khi) in b] for (lo, hi) in b]


def test_pair_weights_are_the_attention_mass_per_partition():
    w = RAGGED
    Q, K, V = _head(w)
    b, st = _slot_states(w, Q, K, V)
    slot_lse = [[st[q][k][1] for k in range(w.P)] for q in range(w.P)]
    merged = [compose(st[q])[1] for q in range(w.P)]
    W = pair_weights(slot_lse, merged)
    # brute force: softmax over all keys, mass on each partition, mean over rows
    z = (Q @ K.T) / math.sqrt(w.d)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for q, (lo, hi) in enumerate(b):
        for k, (klo, khi) in enumerate(b):
            assert W[q, k] == pytest.approx(p[lo:hi, klo:khi].sum(axis=1).mean(), rel=1e-12, abs=1e-15)
        assert W[q].sum() == pytest.approx(1.0, abs=1e-12)


def test_pair_signature_is_mean_restricted_attention():
    w = RAGGED
    Q, K, V = _head(w)
    b, st = _slot_states(w, Q, K, V)
    q, k = 3, 1   # ragged query partition
    (lo, hi), (klo, khi) = b[q], b[k]
    z = (Q[lo:hi] @ K[klo:khi].T) / math.sqrt(w.d)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(pair_signature(st[q][k][0]), (p @ V[klo:khi]).mean(axis=0), atol=1e-13)


def test_drift_and_threshold_closed_forms():
    assert rel_drift([3.0, 4.0], [0.0, 5.0]) == pytest.approx(math.sqrt(10) / 5)
    assert rel_drift([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert rel_drift([1.0], [0.0]) == math.inf
    assert rel_drift([[1.0, 2.0], [3.0, 4.0]], [[1.0, 2.0], [3.0, 4.0]]) == 0.0
    v = [0.3, 0.1, 0.2, 0.4]
    assert reuse_threshold(v, 0.0) == -math.inf
    assert reuse_threshold(v, 0.25) == 0.1
    assert reuse_threshold(v, 0.5) == 0.2
    assert reuse_threshold(v, 0.6) == 0.3     # ceil(2.4) = 3
    assert reuse_threshold(v, 1.0) == 0.4
    assert reuse_threshold([], 0.5) == math.inf


def test_group_members():
    assert group_members(4, 2, 0, 0) == [1] and group_members(4, 2, 0, 1) == [2, 3]
    assert group_members(5, 2, 4, 2) == [] and group_members(5, 2, 3, 2) == [4]
    assert group_members(4, 1, 2, 2) == []


def _sig(P, local, pairs=None):
    """[1][P][P][2] signatures: local[q] on the diagonal, pairs[(q, k)] elsewhere (default [1, 0])."""
    s = np.zeros((1, P, P, 2))
    for q in range(P):
        for k in range(P):
            s[0, q, k] = local[q] if q == k else (pairs or {}).get((q, k), [1.0, 0.0])
    return s


def test_planner_hand_worked_scenario():
    P, g = 4, 2
    pl = AnchorPlanner(P, g, target_reuse=0.5, drift_max=0.9)
    ones = np.ones((P, P), np.uint8)
    Wh = np.full((1, P, P), 0.25)                 # uniform importance
    # step 0: warm-up anchor, nothing cached before
    m, a = pl.plan(0, _sig(P, [[1.0, 0.0]] * P))
    assert a and (m == ones).all()
    s0 = _sig(P, [[1.0, 0.0]] * P)
    pl.update(0, m, Wh, s0, None)
    assert pl.eps == math.inf and (pl.alpha == 0).all()
    # step 1: warm-up anchor; local drift 0.5 everywhere; pair (q, k) drift e = 0.1 * (k + 1)
    loc1 = [[1.0, 0.5]] * P
    m, a = pl.plan(1, _sig(P, loc1))
    assert a and (m == ones).all()
    np.testing.assert_allclose(pl.D, 0.5)
    pairs1 = {(q, k): [1.0, 0.1 * (k + 1)] for q in range(P) for k in range(P) if q != k}
    s1 = _sig(P, loc1, pairs1)
    pl.update(1, m, Wh, s1, s0)
    # alpha = e / D = 0.2 (k + 1);  E(q, G) = 0.25 * sum of member e
    for q in range(P):
        for k in range(P):
            if k != q:
                assert pl.alpha[q, k] == pytest.approx(0.2 * (k + 1))
    # groups with members: q0: {1}, {2,3}; q1: {0}, {2,3}; q2: {0,1}, {3}; q3: {0,1}, {2}
    # E: q0 {1}: .05, {2,3}: .175; q1 {0}: .025, {2,3}: .175; q2 {0,1}: .075, {3}: .1;
    #    q3 {0,1}: .075, {2}: .075  -> sorted .025 .05 .075 .075 .1 .175 .175 (+ .075) ; n = 8
    # rho = .5 -> 4th smallest = .075
    assert pl.eps == pytest.approx(0.075)
    # step 2: local drift against the step-1 reference: q0 0.2, q1 0.05, q2 0.3, q3 0 -> no anchor
    loc2 = [[1.0, 0.5 + 0.2 * math.hypot(1, 0.5)], [1.0, 0.5 + 0.05 * math.hypot(1, 0.5)],
            [1.0, 0.5 + 0.3 * math.hypot(1, 0.5)], [1.0, 0.5]]
    m, a = pl.plan(2, _sig(P, loc2))
    assert not a
    np.testing.assert_allclose(pl.D, [0.2, 0.05, 0.3, 0.0], atol=1e-12)
    # ASE = 0.25 * D * sum of member alpha:
    #   q0: {1} .25*.2*.4 = .02 -> reuse; {2,3} .25*.2*(.6+.8) = .07 -> reuse (<= .075)
    #   q1: {0} .25*.05*.2 -> reuse; {2,3} .25*.05*1.4 = .0175 -> reuse
    #   q2: {0,1} .25*.3*(.2+.4) = .045 -> reuse; {3} .25*.3*.8 = .06 -> reuse
    #   q3: D = 0 -> reuse all
    assert (m == np.eye(P, dtype=np.uint8)).all()
    pl.update(2, m, Wh, _sig(P, loc2, pairs1))
    assert (pl.Dc == 0).all()
    # step 3: q0 drifts to 0.4 -> {2,3}: .25*.4*1.4 = .14 > .075 computed, {1}: .04 reused
    loc3 = [[1.0, 0.5 + 0.4 * math.hypot(1, 0.5)], [1.0, 0.5], [1.0, 0.5], [1.0, 0.5]]
    m, a = pl.plan(3, _sig(P, loc3))
    assert not a
    exp = np.eye(P, dtype=np.uint8)
    exp[0, 2] = exp[0, 3] = 1
    assert (m == exp).all()
    pl.update(3, m, Wh, _sig(P, loc3, pairs1))
    assert pl.Dc[0, 1] == pytest.approx(0.4) and pl.Dc[0, 0] == 0.0
    # step 4: q0 at 0.5 -> {2,3} grows only by 0.1: .25*.1*1.4 = .035 reused; {1}: .25*.5*.4 = .05 reused
    loc4 = [[1.0, 0.5 + 0.5 * math.hypot(1, 0.5)], [1.0, 0.5], [1.0, 0.5], [1.0, 0.5]]
    m, a = pl.plan(4, _sig(P, loc4))
    assert not a and (m == np.eye(P, dtype=np.uint8)).all()
    pl.update(4, m, Wh, _sig(P, loc4, pairs1))
    # step 5: q2 drifts past drift_max -> anchor, everything computed, records reset
    loc5 = [[1.0, 0.5], [1.0, 0.5], [1.0, 0.5 + 0.95 * math.hypot(1, 0.5)], [1.0, 0.5]]
    m, a = pl.plan(5, _sig(P, loc5))
    assert a and (m == ones).all()
    pl.update(5, m, Wh, _sig(P, loc5, pairs1), _sig(P, loc4, pairs1))
    assert (pl.Dc == 0).all() and pl.n_anchors == 3
    assert pl.eps == 0.0      # no pair moved since it was cached: every corrected error is 0


@pytest.mark.parametrize("rho,expect_all", [(0.0, True), (1.0, False)])
def test_planner_unchanged_inputs(rho, expect_all):
    """Signatures that never move: after warm-up there is no drift, so no anchor;
    rho = 0 computes every group (eps = -inf), rho = 1 reuses every group."""
    P, g = 5, 2
    pl = AnchorPlanner(P, g, target_reuse=rho, drift_max=0.0)
    s = _sig(P, [[1.0, 2.0]] * P, {(q, k): [0.5, 0.5] for q in range(P) for k in range(P)})
    W = np.full((2, P, P), 1.0 / P)
    prev = None
    for t in range(6):
        m, a = pl.plan(t, s)
        assert a == (t < 2)
        if t >= 2:
            want = np.ones((P, P), np.uint8) if expect_all else np.eye(P, dtype=np.uint8)
            assert (m == want).all()
        assert (np.diag(m) == 1).all()
        pl.update(t, m, W, s, prev)
        prev = s


def test_planner_rejects_bad_parameters():
    for args in [(4, 0, 0.5, 0.1), (4, 5, 0.5, 0.1), (4, 2, 1.5, 0.1), (4, 2, 0.5, -1.0)]:
        with pytest.raises(ValueError):
            AnchorPlanner(*args)
    with pytest.raises(ValueError):
        AnchorPlanner(4, 2, 0.5, 0.1, warmup=1)


def _zero_importance_case():
    """P = 3, g = 1 (every other partition is a group of its own).  Pair (0, 2)
    has zero importance and an infinite drift at the anchor (its cached
    signature was zero)."""
    W = np.array([[0.5, 0.5, 0.0], [0.3, 0.5, 0.2], [0.4, 0.1, 0.5]])
    e = np.array([[0.0, 0.2, math.inf], [0.1, 0.0, 0.4], [0.3, 0.5, 0.0]])
    return W, e


def test_planner_zero_importance_adds_no_error():
    W, e = _zero_importance_case()
    pl = AnchorPlanner(3, 1, target_reuse=0.5, drift_max=10.0)
    ones = np.ones((3, 3), np.uint8)
    m, a = pl.plan_drift(0, np.zeros(3))
    pl.update_drift(0, m, W, None)
    m, a = pl.plan_drift(1, np.full(3, 0.5))
    assert a
    pl.update_drift(1, ones, W, e)
    # E: q0 {1} .5*.2 = .1, {2} 0 (zero importance); q1 {0} .03, {2} .08; q2 {0} .12, {1} .05
    # sorted 0 .03 .05 .08 .1 .12, rho = .5 -> the 3rd: .05
    assert pl.eps == pytest.approx(0.05)
    assert math.isinf(pl.alpha[0, 2]) and pl.alpha[0, 1] == pytest.approx(0.4)
    # q0 drifts to .6: {1} .5 * .4 * .6 = .12 > .05 computed; {2} has zero importance: reused
    m, a = pl.plan_drift(2, np.array([0.6, 0.0, 0.0]))
    assert not a
    exp = np.eye(3, dtype=np.uint8)
    exp[0, 1] = 1
    assert (m == exp).all()


def test_planner_no_growth_with_infinite_alpha():
    """rho = 0 computes every group: also one whose alpha is +inf while its
    local drift has not grown (no growth predicts no error, 0 > -inf)."""
    W, e = _zero_importance_case()
    W = np.full((3, 3), 1 / 3)
    pl = AnchorPlanner(3, 1, target_reuse=0.0, drift_max=10.0)
    m, _ = pl.plan_drift(0, np.zeros(3))
    pl.update_drift(0, m, W, None)
    m, _ = pl.plan_drift(1, np.full(3, 0.5))
    pl.update_drift(1, m, W, e)
    assert pl.eps == -math.inf and math.isinf(pl.alpha[0, 2])
    m, a = pl.plan_drift(2, np.zeros(3))
    assert not a and m.all()


@pytest.mark.parametrize("what", ["W", "e"])
def test_planner_rejects_nan_statistics(what):
    W, e = _zero_importance_case()
    pl = AnchorPlanner(3, 1, target_reuse=0.5, drift_max=10.0)
    m, _ = pl.plan_drift(0, np.zeros(3))
    pl.update_drift(0, m, W, None)
    m, _ = pl.plan_drift(1, np.full(3, 0.5))
    if what == "W":
        W = W.copy()
        W[1, 2] = math.nan
    else:
        e = e.copy()
        e[2, 0] = math.nan
    with pytest.raises(ValueError):
        pl.update_drift(1, m, W, e)
    assert pl.n_anchors == 1


def test_planner_zero_importance_member_at_rho_zero():
    """rho = 0 (eps = -inf) computes every group, also one whose only member
    has zero importance and an infinite alpha: its ASE is 0, not 0 * inf."""
    W, e = _zero_importance_case()
    pl = AnchorPlanner(3, 1, target_reuse=0.0, drift_max=10.0)
    m, _ = pl.plan_drift(0, np.zeros(3))
    pl.update_drift(0, m, W, None)
    m, _ = pl.plan_drift(1, np.full(3, 0.5))
    pl.update_drift(1, m, W, e)
    m, a = pl.plan_drift(2, np.array([0.6, 0.0, 0.0]))
    assert not a and m.all()
