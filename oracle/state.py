"""Attention state and its composition, fp64.

DiTango page, attention-state section: for a sequence partition i the
attention state AS(i) is the pair (OUT(i), LSE(i)) for every query row, where
LSE(i) is the log-sum-exp of the query's scaled scores against the keys of
partition i and OUT(i) is the softmax over those keys alone applied to their
values.  The page's display equation is lost in extraction; the plain reading
used here, with softmax scale s (1/sqrt(d) unless stated), is

    LSE(i) = log sum_{j in i} exp(s * q.k_j)
    OUT(i) = sum_{j in i} exp(s * q.k_j - LSE(i)) * v_j

Composition (the same section, Eq. 4, associative and commutative) merges the
states of two disjoint key sets into the state of their union:

    LSE(i+j) = log(exp(LSE(i)) + exp(LSE(j)))
    OUT(i+j) = exp(LSE(i) - LSE(i+j)) * OUT(i) + exp(LSE(j) - LSE(i+j)) * OUT(j)

whose weights exp(LSE - LSE(i+j)) are the normalised weights of the
error-analysis section.  ``compose`` is the n-ary form.
"""
from __future__ import annotations

import numpy as np


def partition_bounds(N: int, P: int) -> list[tuple[int, int]]:
    """P contiguous partitions of S = ceil(N/P) tokens; the last may be short.

    Sequence-wise partitioning as in Ring-CP (DiTango page, introduction).
    Raises ValueError if a partition would be empty.
    """
    if N <= 0 or P <= 0:
        raise ValueError("N and P must be positive")
    S = -(-N // P)
    b = [(p * S, min((p + 1) * S, N)) for p in range(P)]
    if any(lo >= hi for lo, hi in b):
        raise ValueError(f"N={N}, P={P}: partition of {S} tokens leaves an empty partition")
    return b


def partial_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """State (OUT [rows, d], LSE [rows]) of query rows q against keys k, values v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = scale * (q @ k.T)                      # scaled scores [rows, keys]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    lse = m[:, 0] + np.log(e.sum(axis=1))
    out = np.exp(z - lse[:, None]) @ v
    return out, lse


def compose2(a, b):
    """Eq. 4: state of the union of two disjoint key sets."""
    oa, la = a
    ob, lb = b
    m = np.maximum(la, lb)
    lse = m + np.log(np.exp(la - m) + np.exp(lb - m))
    out = np.exp(la - lse)[:, None] * oa + np.exp(lb - lse)[:, None] * ob
    return out, lse


def compose(states):
    """n-ary composition of states over disjoint key sets (summed in list order)."""
    states = list(states)
    if not states:
        raise ValueError("compose needs at least one state")
    lses = np.stack([np.asarray(s[1], dtype=np.float64) for s in states])  # [n, rows]
    m = lses.max(axis=0)
    lse = m + np.log(np.exp(lses - m).sum(axis=0))
    out = np.zeros_like(np.asarray(states[0][0], dtype=np.float64))
    for o, l in states:
        out = out + np.exp(np.asarray(l, dtype=np.float64) - lse)[:, None] * o
    return out, lse
