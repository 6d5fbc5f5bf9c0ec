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
from oracle.planner import AnchorPlanner


def _drive(P, g, H, d, rho, drift_max, steps, seed, warmup=2):
    rng = np.random.default_rng(seed)
    rho32, dm32 = float(np.float32(rho)), float(np.float32(drift_max))
    cpp = lib.Planner(P, g, H, d, rho32, dm32, warmup)
    orc = AnchorPlanner(P, g, rho32, dm32, warmup)
    truth = rng.normal(size=(H, P, P, d)).astype(np.float32)        # states the inputs would give now
    rate = rng.uniform(0.0, 0.2, size=(1, P, P, 1)).astype(np.float32)
    table = truth.copy()                                              # signatures of the cached states
    anchors = 0
    for t in range(steps):
        truth = (truth + rate * rng.normal(size=truth.shape)).astype(np.float32)
        before = table.copy()
        for q in range(P):                       # the local states are computed first
            table[:, q, q] = truth[:, q, q]
        sig_local = table.copy()
        m_c, a_c = cpp.plan(t, sig_local)
        m_o, a_o = orc.plan(t, sig_local)
        assert a_c == a_o, (t, seed)
        assert (m_c == m_o).all(), (t, seed, m_c, m_o)
        assert (np.diag(m_c) == 1).all()
        anchors += a_c
        for q in range(P):
            for k in range(P):
                if m_c[q, k]:
                    table[:, q, k] = truth[:, q, k]
        W = rng.dirichlet(np.ones(P), size=(H, P)).astype(np.float32)
        old = None if t == 0 else sig_local
        cpp.update(t, m_c, W, table, old)
        orc.update(t, m_c, W, table, old)
        pl = cpp.pl
        if math.isinf(orc.eps):
            assert math.isinf(pl.eps) and (pl.eps > 0) == (orc.eps > 0)
        else:
            assert pl.eps == pytest.approx(orc.eps, rel=1e-12, abs=1e-300)
        np.testing.assert_allclose(np.array(pl.D)[:P], orc.D, rtol=1e-12, atol=0)
        np.testing.assert_allclose(np.array([row[:P] for row in pl.alpha])[:P], orc.alpha, rtol=1e-12, atol=0)
        np.testing.assert_allclose(np.array([row[:orc.m] for row in pl.Dc])[:P], orc.Dc, rtol=1e-12, atol=0)
        assert pl.n_anchors == orc.n_anchors
        del before
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


def test_planner_rejects_bad_arguments():
    ref = np.zeros((2, 4, 4), np.float32)
    pl = binding.ditango_planner_t()
    f = binding._f32(ref)
    init = binding.lib.ditango_planner_init
    assert init(ctypes.byref(pl), 4, 2, 2, 4, 0.5, 0.1, 2, f) == lib.DITANGO_OK
    for args in [(0, 2, 2, 4, 0.5, 0.1, 2), (33, 2, 2, 4, 0.5, 0.1, 2), (4, 0, 2, 4, 0.5, 0.1, 2),
                 (4, 5, 2, 4, 0.5, 0.1, 2), (4, 2, 0, 4, 0.5, 0.1, 2), (4, 2, 2, 4, 1.5, 0.1, 2),
                 (4, 2, 2, 4, 0.5, -0.1, 2), (4, 2, 2, 4, 0.5, 0.1, 1)]:
        assert init(ctypes.byref(pl), *args, f) == lib.DITANGO_EINVAL, args
    assert init(ctypes.byref(pl), 4, 2, 2, 4, 0.5, 0.1, 2, None) == lib.DITANGO_EINVAL
    # an uninitialised planner is refused
    blank = binding.ditango_planner_t()
    mask = np.zeros((4, 4), np.uint8)
    sig = np.zeros((2, 4, 4, 4), np.float32)
    assert binding.lib.ditango_planner_plan(ctypes.byref(blank), 0, binding._f32(sig), binding._u8(mask),
                                            None) == lib.DITANGO_EINVAL
    assert binding.lib.ditango_last_error()
