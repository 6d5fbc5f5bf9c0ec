"""Pins of the oracle's selective compute-and-reuse step (CPU only).

Special cases the DiTango page fixes: reusing every state reproduces the
cached step; with unchanged inputs reuse is exact; t_c is the last step a
pair was computed and anchors reset it; the grouped form of Fig. 6 (compose
the remote states, cache the composite) gives the same output as reusing the
pairs one by one.
"""
import math

import numpy as np
import pytest

import synth
from oracle.masks import all_fresh, all_reuse, radius_mask, step_mask
from oracle.reuse import ReuseError, StateReuseOracle, run_workload
from oracle.state import compose, compose2, partial_state, partition_bounds

SMALL = synth.get("tiny").scaled(name="tiny_small", F=2, Hh=6, W=7, H=2, d=8, P=4, steps=4)


def _inputs(w, t):
    q, k, v = synth.step_inputs(w, t)
    return {h: (synth.bf16_bits_to_f64(q[h]), synth.bf16_bits_to_f64(k[h]), synth.bf16_bits_to_f64(v[h]))
            for h in range(w.H)}


def test_all_reuse_reproduces_cached_step():
    w = SMALL
    orc = StateReuseOracle(w.N, w.P, w.d)
    r0 = orc.step(0, all_fresh(w.P), _inputs(w, 0))
    r1 = orc.step(1, all_reuse(w.P), _inputs(w, 1))
    for h in range(w.H):
        np.testing.assert_allclose(r1["O"][h], r0["O"][h], atol=1e-12)
        np.testing.assert_allclose(r1["LSE"][h], r0["LSE"][h], atol=1e-12)
    assert r1["fresh"] == {}
    assert np.all(r1["tc"] == 0)


def test_zero_drift_makes_any_mask_exact():
    w = SMALL.scaled(sigma=0.0)
    ref = StateReuseOracle(w.N, w.P, w.d).step(0, all_fresh(w.P), _inputs(w, 0))
    orc = StateReuseOracle(w.N, w.P, w.d)
    orc.step(0, all_fresh(w.P), _inputs(w, 0))
    rng = np.random.default_rng(0)
    for t in range(1, 4):
        m = (rng.random((w.P, w.P)) < 0.4).astype(np.uint8)
        r = orc.step(t, m, _inputs(w, t))
        for h in range(w.H):
            np.testing.assert_allclose(r["O"][h], ref["O"][h], atol=1e-12)
            np.testing.assert_allclose(r["LSE"][h], ref["LSE"][h], atol=1e-12)


def test_reuse_takes_state_from_last_fresh_step():
    """t_c semantics: a pair reused at t carries the state computed at t_c."""
    w = SMALL
    P = w.P
    orc = StateReuseOracle(w.N, P, w.d)
    orc.step(0, all_fresh(P), _inputs(w, 0))
    m1 = radius_mask(P, 1)
    orc.step(1, m1, _inputs(w, 1))
    m2 = radius_mask(P, 0)
    orc.step(2, m2, _inputs(w, 2))
    want_tc = np.zeros((P, P), int)
    want_tc[m1 == 1] = 1
    want_tc[m2 == 1] = 2
    assert np.array_equal(orc.tc, want_tc)
    # pair (0, 1) was fresh at step 1 and reused at step 2: its cached state
    # must be the step-1 state, recomputed here from step-1 inputs
    x1 = _inputs(w, 1)[0]
    lo0, hi0 = partition_bounds(w.N, P)[0]
    lo1, hi1 = partition_bounds(w.N, P)[1]
    want = partial_state(x1[0][lo0:hi0], x1[1][lo1:hi1], x1[2][lo1:hi1], 1 / math.sqrt(w.d))
    got = orc.cache[(0, 0, 1)]
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    # pair (0, 3) was last fresh at the anchor
    x0 = _inputs(w, 0)[0]
    lo3, hi3 = partition_bounds(w.N, P)[3]
    want0 = partial_state(x0[0][lo0:hi0], x0[1][lo3:hi3], x0[2][lo3:hi3], 1 / math.sqrt(w.d))
    np.testing.assert_array_equal(orc.cache[(0, 0, 3)][0], want0[0])


def test_reuse_of_never_computed_pair_is_refused():
    w = SMALL
    orc = StateReuseOracle(w.N, w.P, w.d)
    with pytest.raises(ReuseError):
        orc.step(0, radius_mask(w.P, 1), _inputs(w, 0))
    assert np.all(orc.tc == -1) and orc.cache == {}


def test_anchor_mid_run_resets_tc():
    w = SMALL
    orc = StateReuseOracle(w.N, w.P, w.d)
    orc.step(0, all_fresh(w.P), _inputs(w, 0))
    orc.step(1, radius_mask(w.P, 1), _inputs(w, 1))
    orc.step(2, all_fresh(w.P), _inputs(w, 2))
    assert np.all(orc.tc == 2)


def test_fig6_grouped_reuse_equals_per_pair_reuse():
    """Fig. 6: at t-1 compose AS(2), AS(3) and cache AS(2+3); at t compute AS(0),
    AS(1) fresh and compose with the cached composite.  The per-pair cache
    with mask row [1 1 0 0] must give the same output for query partition 0."""
    w = SMALL
    P, s = w.P, 1 / math.sqrt(w.d)
    b = partition_bounds(w.N, P)
    x0, x1 = _inputs(w, 0)[0], _inputs(w, 1)[0]
    lo, hi = b[0]
    st = lambda x, k: partial_state(x[0][lo:hi], x[1][b[k][0]:b[k][1]], x[2][b[k][0]:b[k][1]], s)
    cached_23 = compose2(st(x0, 2), st(x0, 3))
    fig6 = compose([st(x1, 0), st(x1, 1), cached_23])
    orc = StateReuseOracle(w.N, P, w.d)
    orc.step(0, all_fresh(P), {0: x0})
    r = orc.step(1, radius_mask(P, 1), {0: x1})
    np.testing.assert_allclose(r["O"][0][lo:hi], fig6[0], atol=1e-13)
    np.testing.assert_allclose(r["LSE"][0][lo:hi], fig6[1], atol=1e-13)


def test_sampled_rows_match_full_run():
    """Tracking a subset of query rows gives those rows of the full run (up to
    the BLAS blocking of a shorter matrix product)."""
    w = SMALL
    rows = np.array([0, 5, 17, 40, w.N - 1])
    full = run_workload(w)
    samp = run_workload(w, rows=rows)
    for h in range(w.H):
        np.testing.assert_allclose(samp["O"][h], full["O"][h][rows], atol=1e-14, rtol=0)
        np.testing.assert_allclose(samp["LSE"][h], full["LSE"][h][rows], atol=1e-14, rtol=0)


def test_partial_reuse_lies_between_fresh_and_stale():
    """Sanity of the approximation on the tiny workload: reusing the far states
    from one step back is closer to the all-fresh step-1 output than reusing
    every state (the step-0 output) is, and it is not exact."""
    w = synth.get("tiny").scaled(H=1)
    fresh = run_workload(w, masks={1: all_fresh(w.P)})
    reuse = run_workload(w)
    stale = run_workload(w, masks={1: all_reuse(w.P)})
    err = np.abs(fresh["O"][0] - reuse["O"][0]).mean()
    err_stale = np.abs(fresh["O"][0] - stale["O"][0]).mean()
    assert 0 < err < 0.5 * err_stale
    assert np.array_equal(reuse["reused"], (step_mask(w, 1) == 0).astype(np.uint8))
