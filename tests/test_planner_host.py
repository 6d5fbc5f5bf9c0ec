"""The library's planner (host C++, ditango_planner_*) against the oracle
planner on identical statistics (CPU only: the planner does no device work).

Both take their decisions in double precision from the same float32 inputs,
so masks and anchor decisions must be identical and eps, alpha and the
per-group records equal to rounding.
"""
import ctypes
import math

import numpy as np
import pytest

import context_state_reuse_amd as lib
from context_state_reuse_amd import binding
from oracle.planner import AnchorPlanner, rel_drift


def _drive(P, g, H, d, rho, drift_max, steps, seed, warmup=2):
    """Signatures evolve at pair-specific rates; the drifts the planner needs
    are computed once (float32, as the GPU reductions deliver them) and fed
    to both planners."""
    rng = np.random.default_rng(seed)
    rho32, dm32 = float(np.float32(rho)), float(np.float32(drift_max))
    cpp = lib.Planner(P, g, H, rho32, dm32, warmup)
    orc = AnchorPlanner(P, g, rho32, dm32, warmup)
    truth = rng.normal(size=(H, P, P, d)).astype(np.float32)        # states the inputs would give now
    rate = rng.uniform(0.0, 0.2, size=(1, P, P, 1)).astype(np.float32)
    table = truth.copy()                                              # signatures of the cached states
    ref = None                                                        # signatures at the last anchor
    anchors = 0
    for t in range(steps):
        truth = (truth + rate * rng.normal(size=truth.shape)).astype(np.float32)
        for q in range(P):                       # the local states are computed first
            table[:, q, q] = truth[:, q, q]
        D = None if ref is None else np.array([rel_drift(table[:, q, q], ref[:, q, q]) for q in range(P)],
                                              dtype=np.float32)
        m_c, a_c = cpp.plan(t, D)
        m_o, a_o = orc.plan_drift(t, D if D is not None else np.zeros(P))
        assert a_c == a_o, (t, seed)
        assert (m_c == m_o).all(), (t, seed, m_c, m_o)
        assert (np.diag(m_c) == 1).all()
        anchors += a_c
        old = table.copy()
        for q in range(P):
            for k in range(P):
                if m_c[q, k]:
                    table[:, q, k] = truth[:, q, k]
        W = rng.dirichlet(np.ones(P), size=(H, P)).astype(np.float32)
        if a_c:
            e = None if ref is None else np.array([[rel_drift(table[:, q, k], old[:, q, k]) if k != q else 0.0
                                                    for k in range(P)] for q in range(P)], dtype=np.float32)
            cpp.update(t, m_c, W, e)
            orc.update_drift(t, m_c, np.mean(W.astype(np.float64), axis=0), e)
            ref = table.copy()
        else:
            cpp.update(t, m_c)
            orc.update_drift(t, m_c, None, None)
        pl = cpp.pl
        if math.isinf(orc.eps):
            assert math.isinf(pl.eps) and (pl.eps > 0) == (orc.eps > 0)
        else:
            assert pl.eps == pytest.approx(orc.eps, rel=1e-12, abs=1e-300)
        np.testing.assert_allclose(np.array(pl.D)[:P], orc.D, rtol=1e-12, atol=0)
        np.testing.assert_allclose(np.array([row[:P] for row in pl.alpha])[:P], orc.alpha, rtol=1e-12, atol=0)
        np.testing.assert_allclose(np.array([row[:orc.m] for row in pl.Dc])[:P], orc.Dc, rtol=1e-12, atol=0)
        assert pl.n_anchors == orc.n_anchors
    return anchors


@pytest.mark.parametrize("P,g,rho,drift_max,seed", [
    (4, 2, 0.5, 0.3, 1), (5, 2, 0.75, 0.5, 2), (8, 3, 0.6, 0.4, 3), (8, 1, 0.9, 1.0, 4),
    (6, 6, 0.5, 0.2, 5), (3, 2, 0.0, 0.5, 6), (7, 2, 1.0, 0.5, 7), (32, 4, 0.7, 0.6, 8)])
def test_library_planner_matches_oracle(P, g, rho, drift_max, seed):
    anchors = _drive(P, g, 2, 4, rho, drift_max, 12, seed)
    assert 2 <= anchors <= 12


def test_library_planner_mixes_anchor_and_selective_steps():
    # slow drift and a loose bound: anchors only at warm-up, then selective steps
    anchors = _drive(8, 2, 3, 8, 0.5, 5.0, 10, 11)
    assert anchors == 2


def test_planner_single_partition_has_no_groups():
    # P = 1: the only pair is the local one, always computed; no group ever decides anything
    pl = lib.Planner(1, 1, 2, 0.5, 0.1)
    orc = AnchorPlanner(1, 1, 0.5, float(np.float32(0.1)))
    for t in range(5):
        D = None if t == 0 else np.array([0.05 * t], np.float32)
        m, a = pl.plan(t, D)
        mo, ao = orc.plan_drift(t, D if D is not None else np.zeros(1))
        assert m.tolist() == [[1]] and a == ao and (mo == m).all()
        W = np.ones((2, 1, 1), np.float32)
        e = None if t == 0 else np.zeros((1, 1), np.float32)
        pl.update(t, m, W if a else None, e if a else None)
        orc.update_drift(t, m, np.ones((1, 1)) if a else None, e if a else None)
        assert pl.eps == orc.eps


def test_planner_nan_drift_forces_an_anchor():
    pl = lib.Planner(4, 2, 1, 0.5, 10.0)
    for t in range(2):
        m, a = pl.plan(t, None if t == 0 else np.zeros(4, np.float32))
        pl.update(t, m, np.full((1, 4, 4), 0.25, np.float32), None if t == 0 else np.zeros((4, 4), np.float32))
    m, a = pl.plan(2, np.array([0.0, np.nan, 0.0, 0.0], np.float32))
    assert a and m.all()


def test_planner_rejects_bad_arguments():
    pl = binding.ditango_planner_t()
    init = binding.lib.ditango_planner_init
    assert init(ctypes.byref(pl), 4, 2, 2, 0.5, 0.1, 2) == lib.DITANGO_OK
    for args in [(0, 2, 2, 0.5, 0.1, 2), (33, 2, 2, 0.5, 0.1, 2), (4, 0, 2, 0.5, 0.1, 2), (4, 5, 2, 0.5, 0.1, 2),
                 (4, 2, 0, 0.5, 0.1, 2), (4, 2, 2, 1.5, 0.1, 2), (4, 2, 2, 0.5, -0.1, 2), (4, 2, 2, 0.5, 0.1, 1)]:
        assert init(ctypes.byref(pl), *args) == lib.DITANGO_EINVAL, args
    assert init(None, 4, 2, 2, 0.5, 0.1, 2) == lib.DITANGO_EINVAL
    # an uninitialised planner is refused; drift is required after the first anchor
    blank = binding.ditango_planner_t()
    mask = np.zeros((4, 4), np.uint8)
    assert binding.lib.ditango_planner_plan(ctypes.byref(blank), 0, None, binding._u8(mask), None) == lib.DITANGO_EINVAL
    assert binding.lib.ditango_last_error()
    p = lib.Planner(4, 2, 1, 0.5, 0.1)
    m, a = p.plan(0, None)
    with pytest.raises(lib.DitangoError):
        p.update(0, m, None, None)                    # W is required at an anchor
    p.update(0, m, np.full((1, 4, 4), 0.25, np.float32))
    with pytest.raises(lib.DitangoError):
        p.plan(1, None)                               # drift is required after the first anchor


def _zero_importance_inputs():
    # importance per head (2 heads, same mean as the oracle pin's case)
    Wm = np.array([[0.5, 0.5, 0.0], [0.3, 0.5, 0.2], [0.4, 0.1, 0.5]], np.float32)
    e = np.array([[0.0, 0.2, np.inf], [0.1, 0.0, 0.4], [0.3, 0.5, 0.0]], np.float32)
    return np.stack([Wm, Wm]), e


@pytest.mark.parametrize("rho", [0.0, 0.5, 1.0])
def test_library_planner_zero_importance_and_infinite_drift(rho):
    W, e = _zero_importance_inputs()
    cpp = lib.Planner(3, 1, 2, rho, 10.0)
    orc = AnchorPlanner(3, 1, rho, 10.0)
    for t, D in enumerate([None, [0.5] * 3, [0.6, 0.0, 0.0], [0.0] * 3, [0.9, 0.7, 0.2]]):
        Dv = None if D is None else np.array(D, np.float32)
        m_c, a_c = cpp.plan(t, Dv)
        m_o, a_o = orc.plan_drift(t, Dv if Dv is not None else np.zeros(3))
        assert a_c == a_o and (m_c == m_o).all(), (t, m_c, m_o)
        if a_c:
            cpp.update(t, m_c, W, None if t == 0 else e)
            orc.update_drift(t, m_c, W.mean(axis=0).astype(np.float64), None if t == 0 else e)
        else:
            cpp.update(t, m_c)
            orc.update_drift(t, m_c, None, None)
        assert cpp.pl.eps == orc.eps or (math.isinf(cpp.pl.eps) and cpp.pl.eps == orc.eps)


@pytest.mark.parametrize("what", ["W", "e", "e_negative"])
def test_library_planner_rejects_nan_statistics_unchanged(what):
    W, e = _zero_importance_inputs()
    p = lib.Planner(3, 1, 2, 0.5, 10.0)
    m, _ = p.plan(0, None)
    p.update(0, m, W)
    m, a = p.plan(1, np.full(3, 0.5, np.float32))
    assert a
    if what == "W":
        W = W.copy()
        W[1, 0, 2] = np.nan
    elif what == "e":
        e = e.copy()
        e[2, 0] = np.nan
    else:
        e = e.copy()
        e[1, 2] = -0.5
    before = bytes(p.pl)
    with pytest.raises(lib.DitangoError):
        p.update(1, m, W, e)
    assert bytes(p.pl) == before                      # nothing changed
    p.update(1, m, *_zero_importance_inputs())        # valid statistics are still taken
    assert p.pl.n_anchors == 2
