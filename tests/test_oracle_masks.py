"""Pins of the oracle's selection masks and its SplitMix64 (CPU only)."""
import os

import numpy as np
import pytest

import synth
from oracle.masks import (SplitMix64, nearest_mask, radius_mask, random_mask,
                          step_mask)


def _read_golden(path):
    with open(path) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_splitmix64_published_vectors(golden_dir):
    for line in _read_golden(os.path.join(golden_dir, "splitmix64_vectors.txt")):
        seed, outs = line.split(":")
        rng = SplitMix64(int(seed))
        for want in outs.split():
            assert rng.next() == int(want, 0)


def test_fig6_example_row(golden_dir):
    """CP = 4, rank 0 (Fig. 6): partitions 0 and 1 fresh, 2 and 3 reused."""
    g = dict(ln.split(":") for ln in _read_golden(os.path.join(golden_dir, "fig6_cp4_rank0.txt")))
    P, q = int(g["P"]), int(g["query_partition"])
    m = radius_mask(P, 1)
    assert sorted(np.flatnonzero(m[q])) == [int(x) for x in g["fresh"].split()]
    assert sorted(np.flatnonzero(m[q] == 0)) == [int(x) for x in g["reused"].split()]


def test_tiny_step1_mask(golden_dir):
    want = np.array([[int(x) for x in ln.split()]
                     for ln in _read_golden(os.path.join(golden_dir, "tiny_step1_mask.txt"))], np.uint8)
    assert np.array_equal(step_mask(synth.get("tiny"), 1), want)
    assert want.sum(1).tolist() == [2, 3, 3, 2]


def test_step0_is_anchor():
    for w in synth.WORKLOADS.values():
        assert np.array_equal(step_mask(w, 0), np.ones((w.P, w.P), np.uint8))


def test_nearest_tie_break_lower_index():
    m2 = nearest_mask(8, 2)
    assert sorted(np.flatnonzero(m2[0])) == [0, 1]
    assert sorted(np.flatnonzero(m2[3])) == [2, 3]
    assert sorted(np.flatnonzero(m2[7])) == [6, 7]
    m4 = nearest_mask(8, 4)
    assert sorted(np.flatnonzero(m4[3])) == [1, 2, 3, 4]
    assert sorted(np.flatnonzero(m4[0])) == [0, 1, 2, 3]
    m4_16 = nearest_mask(16, 4)
    assert sorted(np.flatnonzero(m4_16[5])) == [3, 4, 5, 6]
    # nearest-n is not symmetric in general
    assert not np.array_equal(m2, m2.T)


@pytest.mark.parametrize("name,count", [("image", 2), ("video_100", 8), ("video_50", 4),
                                        ("video_25", 2), ("long", 4), ("stress", 8)])
def test_row_counts_and_diagonal(name, count):
    w = synth.get(name)
    for t in range(1, w.steps):
        m = step_mask(w, t)
        assert m.sum(1).tolist() == [count] * w.P
        assert np.all(np.diag(m) == 1)


def test_random_mask_varies_by_step_and_is_seeded():
    w = synth.get("stress")
    masks = [step_mask(w, t) for t in range(1, w.steps)]
    assert len({m.tobytes() for m in masks}) == len(masks)
    assert np.array_equal(step_mask(w, 3), random_mask(32, 8, 5003))
    assert masks[0].sum() == 256


def test_random_mask_small_by_hand():
    """P = 4, n = 2: per row, self plus c[j] with j = next() mod 3 from c = [k != q]."""
    rng = SplitMix64(77)
    want = np.zeros((4, 4), np.uint8)
    for q in range(4):
        c = [k for k in range(4) if k != q]
        want[q, q] = 1
        want[q, c[rng.next() % 3]] = 1
    assert np.array_equal(random_mask(4, 2, 77), want)


def test_random_mask_several_swaps_by_hand():
    """Rows whose draws are the published SplitMix64 check values (golden
    file), with two and three swaps per row, worked by hand:

    seed 0, P = 5, n = 3 (draws o0..o3; candidates of row q are [k != q]):
      row 0: c = [1, 2, 3, 4]; o0 mod 4 = 3 -> swap c[0], c[3] -> [4, 2, 3, 1];
             o1 mod 3 = 0 -> j = 1, no swap; fresh = {0} + {4, 2}
      row 1: c = [0, 2, 3, 4]; o2 mod 4 = 3 -> [4, 2, 3, 0];
             o3 mod 3 = 1 -> j = 2 -> swap c[1], c[2] -> [4, 3, 2, 0];
             fresh = {1} + {4, 3}
    seed 1234567, P = 5, n = 4 (draws d0..d2):
      row 0: c = [1, 2, 3, 4]; d0 mod 4 = 1 -> [2, 1, 3, 4];
             d1 mod 3 = 1 -> j = 2 -> [2, 3, 1, 4]; d2 mod 2 = 1 -> j = 3 ->
             [2, 3, 4, 1]; fresh = {0} + {2, 3, 4}
    A modulus of P-1 at every swap, a dropped "+ i", or taking c[1..n-1]
    changes at least one of these rows.
    """
    m = random_mask(5, 3, 0)
    assert np.flatnonzero(m[0]).tolist() == [0, 2, 4]
    assert np.flatnonzero(m[1]).tolist() == [1, 3, 4]
    m = random_mask(5, 4, 1234567)
    assert np.flatnonzero(m[0]).tolist() == [0, 2, 3, 4]
