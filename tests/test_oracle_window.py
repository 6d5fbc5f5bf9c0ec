"""Pins of the window-attention-with-residual-sharing oracle (CPU only).

Fixed independently of its code: the full step is full softmax attention
(brute force); the cached residual is full attention minus one-shot
attention over the window partitions' keys; a window that covers every
partition leaves no residual; with unchanged inputs a window step returns
the full step's output exactly; and, as the DiTFastAttn page's ablation
reports, adding the residual brings window attention closer to full
attention when inputs drift slowly.
"""
import math

import numpy as np
import pytest

import synth
from oracle.masks import all_fresh, nearest_mask, radius_mask
from oracle.state import partition_bounds
from oracle.window_residual import WindowResidualOracle


def _inputs(w, t, heads=None):
    q, k, v = synth.step_inputs(w, t)
    heads = range(w.H) if heads is None else heads
    return {h: (synth.bf16_bits_to_f64(q[h]), synth.bf16_bits_to_f64(k[h]), synth.bf16_bits_to_f64(v[h]))
            for h in heads}


def _brute(q, k, v, scale):
    z = scale * (q @ k.T)
    lse = np.array([math.log(sum(math.exp(x) for x in row)) for row in z])
    return np.exp(z - lse[:, None]) @ v, lse


RAGGED = synth.get("tiny").scaled(name="tiny_ragged_w", F=1, Hh=1, W=37, H=1, d=8, P=5, steps=3)


def test_full_step_is_full_attention_and_residual_is_full_minus_window():
    w = RAGGED
    x = _inputs(w, 0)
    Q, K, V = x[0]
    win = nearest_mask(w.P, 2)
    orc = WindowResidualOracle(w.N, w.P, w.d)
    r = orc.full_step(win, x)
    s = 1 / math.sqrt(w.d)
    o, l = _brute(Q, K, V, s)
    np.testing.assert_allclose(r["O"][0], o, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][0], l, atol=1e-12)
    b = partition_bounds(w.N, w.P)
    for q in range(w.P):
        keys = np.concatenate([np.arange(*b[k]) for k in range(w.P) if win[q, k]])
        lo, hi = b[q]
        o_win, _ = _brute(Q[lo:hi], K[keys], V[keys], s)
        np.testing.assert_allclose(orc.residual[0][lo:hi], o[lo:hi] - o_win, atol=1e-12)


def test_window_covering_everything_leaves_no_residual():
    w = RAGGED
    orc = WindowResidualOracle(w.N, w.P, w.d)
    orc.full_step(all_fresh(w.P), _inputs(w, 0))
    assert np.abs(orc.residual[0]).max() < 1e-15
    x1 = _inputs(w, 1)
    r = orc.window_step(all_fresh(w.P), x1)
    o, l = _brute(*x1[0], 1 / math.sqrt(w.d))
    np.testing.assert_allclose(r["O"][0], o, atol=1e-12)
    np.testing.assert_allclose(r["LSE"][0], l, atol=1e-12)


@pytest.mark.parametrize("window", ["nearest2", "radius1", "self"])
def test_unchanged_inputs_reproduce_the_full_step(window):
    w = RAGGED.scaled(sigma=0.0)
    win = {"nearest2": nearest_mask(w.P, 2), "radius1": radius_mask(w.P, 1),
           "self": np.eye(w.P, dtype=np.uint8)}[window]
    orc = WindowResidualOracle(w.N, w.P, w.d)
    full = orc.full_step(win, _inputs(w, 0))
    for t in (1, 2):
        r = orc.window_step(win, _inputs(w, t))
        np.testing.assert_allclose(r["O"][0], full["O"][0], atol=1e-12)


def test_residual_sharing_beats_window_alone_under_slow_drift():
    w = synth.get("tiny").scaled(H=1)
    win = radius_mask(w.P, 1)
    x0, x1 = _inputs(w, 0), _inputs(w, 1)
    orc = WindowResidualOracle(w.N, w.P, w.d)
    orc.full_step(win, x0)
    wars = orc.window_step(win, x1)["O"][0]
    full1 = WindowResidualOracle(w.N, w.P, w.d).full_step(win, x1)["O"][0]   # full attention at step 1
    no_res = wars - orc.residual[0]               # window attention alone at step 1
    err_wars = np.abs(wars - full1).mean()
    err_win = np.abs(no_res - full1).mean()
    assert 0 < err_wars < 0.5 * err_win


def test_errors():
    w = RAGGED
    orc = WindowResidualOracle(w.N, w.P, w.d)
    with pytest.raises(RuntimeError):
        orc.window_step(nearest_mask(w.P, 2), _inputs(w, 0))
    empty = nearest_mask(w.P, 2)
    empty[2] = 0
    with pytest.raises(ValueError):
        orc.full_step(empty, _inputs(w, 0))
