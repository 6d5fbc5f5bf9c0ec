"""Per-step COMPUTE/REUSE masks over (query partition, KV partition) pairs.

DiTango page, state-selection section: at each timestep every unit is either
recomputed (COMPUTE) or served from its cached state (REUSE); the spatial
locality study (Fig. 5a) finds near partitions matter most, and anchor steps
force every unit to compute.  Here the unit is one pair (group size 1), the
mask is a P x P uint8 array with mask[q, k] = 1 meaning COMPUTE (fresh) and
0 meaning REUSE, and step 0 is the anchor (all ones).  The workloads replace
the page's error-threshold planner with fixed locality policies:

* ``radius r``  -- fresh iff |q - k| <= r;
* ``nearest n`` -- per query partition q, the n KV partitions with the
  smallest |q - k|, ties broken toward the lower index k (sort by (|q-k|, k));
* ``random n``  -- per q, q itself plus n-1 distinct others drawn with
  SplitMix64 (seed 1000*cfg_id + t): rows in order q = 0..P-1, candidates
  c = [k != q] ascending, for i = 0..n-2 swap c[i] with
  c[i + next() mod (P-1-i)], fresh = {q} + c[0..n-2].

SplitMix64 follows its published definition (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; the mix64 variant
with constants 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB and golden-gamma
increment 0x9E3779B97F4A7C15).
"""
from __future__ import annotations

import numpy as np

_M64 = (1 << 64) - 1


class SplitMix64:
    def __init__(self, seed: int):
        self.state = seed & _M64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _M64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        return z ^ (z >> 31)


def all_fresh(P: int) -> np.ndarray:
    return np.ones((P, P), dtype=np.uint8)


def all_reuse(P: int) -> np.ndarray:
    return np.zeros((P, P), dtype=np.uint8)


def radius_mask(P: int, r: int) -> np.ndarray:
    m = np.zeros((P, P), dtype=np.uint8)
    for q in range(P):
        for k in range(P):
            if abs(q - k) <= r:
                m[q, k] = 1
    return m


def nearest_mask(P: int, n: int) -> np.ndarray:
    if not 1 <= n <= P:
        raise ValueError("need 1 <= n <= P")
    m = np.zeros((P, P), dtype=np.uint8)
    for q in range(P):
        order = sorted(range(P), key=lambda k: (abs(q - k), k))
        for k in order[:n]:
            m[q, k] = 1
    return m


def random_mask(P: int, n: int, seed: int) -> np.ndarray:
    if not 1 <= n <= P:
        raise ValueError("need 1 <= n <= P")
    rng = SplitMix64(seed)
    m = np.zeros((P, P), dtype=np.uint8)
    for q in range(P):
        c = [k for k in range(P) if k != q]
        for i in range(n - 1):
            j = i + rng.next() % (P - 1 - i)
            c[i], c[j] = c[j], c[i]
        m[q, q] = 1
        for k in c[:n - 1]:
            m[q, k] = 1
    return m


def policy_mask(policy: str, P: int, n: int, seed: int) -> np.ndarray:
    if policy == "radius":
        return radius_mask(P, n)
    if policy == "nearest":
        return nearest_mask(P, n)
    if policy == "random":
        return random_mask(P, n, seed)
    if policy == "all":
        return all_fresh(P)
    if policy == "none":
        return all_reuse(P)
    raise ValueError(f"unknown mask policy {policy!r}")


def step_mask(w, t: int) -> np.ndarray:
    """Mask of step t of workload w; step 0 is the all-fresh anchor."""
    if t == 0:
        return all_fresh(w.P)
    return policy_mask(w.policy, w.P, w.n_fresh, 1000 * w.cfg_id + t)
