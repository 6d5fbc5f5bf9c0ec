"""Grouped, composed attention-state cache, fp64 (test infrastructure only).

DiTango page, state-selection section: the p partition states of a query
partition are grouped into groups of g spatially adjacent partitions; the
local state is handled on its own, so the group that contains it keeps g - 1
states.  Compute-or-reuse is decided per group, and t_c is kept per group.
Selective compute and reuse (Fig. 6): the states of a group are composed and
the composite is what the cache holds; a reused group contributes that
cached composite.  Ring-based composed attention: a fresh group state is
built over the group's g members, one partial attention per member composed
into the running state with Eq. 4.  Dynamic Group State Compose: when the
cache grows too large, groups are merged k at a time (group size g -> k g)
by composing their cached states; an anchor step recomputes everything at
the original group size.

Readings where the page is silent (each is the plainest one the rest
supports):

* groups are fixed, contiguous and global: G_j = {j g, ..., min((j+1) g, P) - 1},
  j < m = ceil(P / g); for query partition q the state of group j covers
  G_j minus {q}.  A group that is {q} alone holds no state;
* slots of query partition q: slot 0 = the local pair (q, q), slot 1 + j =
  group j;
* the per-step selection arrives as the pair mask of the per-pair form
  (1 = fresh); a group is recomputed when any of its members is marked
  fresh (a composed state can only be refreshed as a whole), the local slot
  follows mask[q][q];
* the members of a fresh group are composed in ascending partition order;
* merging groups: new group i covers old groups k i .. k i + k - 1, its state
  is their composition in ascending order (empty ones skipped) and its t_c
  is the oldest of theirs (the age the error model must assume);
* the row merge composes the live slots in slot order.
"""
from __future__ import annotations

import numpy as np

from .reuse import ReuseError
from .state import compose, compose2, partial_state, partition_bounds


def n_groups(P: int, g: int) -> int:
    return -(-P // g)


def n_slots(P: int, g: int) -> int:
    """Slots per query partition: the local pair plus one per group."""
    return 1 + n_groups(P, g)


def slot_bytes(H: int, N: int, P: int, d: int, out_bytes: int = 4) -> int:
    """Device bytes of one slot of the grouped cache: OUT [H][P][S][d] of
    out_bytes per element (4: fp32, the default; 2: bf16) plus LSE [H][P][S]
    in fp32, the layout the library allocates per slot."""
    S = -(-N // P)
    return H * P * S * (out_bytes * d + 4)


def merges_to_fit(P: int, g: int, k: int, bytes_per_slot: int, budget: int) -> int:
    """Dynamic Group State Compose, memory trigger (DiTango page, dynamic
    group state compose: groups are merged, repeatedly if need be, once the
    cache's memory nears its limit): the number of merges by k after which
    the cache, n_slots(P, g) slots of bytes_per_slot each, fits the budget.
    Raises ValueError when one group of all P partitions does not fit."""
    if k < 2:
        raise ValueError("merge factor must be >= 2")
    n = 0
    while n_slots(P, g) * bytes_per_slot > budget:
        if g >= P:
            raise ValueError("the cache does not fit the budget even as one group")
        g *= k
        n += 1
    return n


def slot_members(P: int, g: int, q: int, s: int) -> list[int]:
    """KV partitions whose composed state slot s of query partition q holds."""
    if s == 0:
        return [q]
    j = s - 1
    return [k for k in range(j * g, min((j + 1) * g, P)) if k != q]


def group_decisions(mask: np.ndarray, g: int) -> np.ndarray:
    """uint8 [P][n_slots]: 1 = slot recomputed this step; empty slots are 0."""
    mask = np.asarray(mask, dtype=np.uint8)
    P = mask.shape[0]
    out = np.zeros((P, n_slots(P, g)), dtype=np.uint8)
    for q in range(P):
        for s in range(n_slots(P, g)):
            mem = slot_members(P, g, q, s)
            out[q, s] = 1 if any(mask[q, k] for k in mem) else 0
    return out


def nearest_groups_mask(P: int, g: int, n: int) -> np.ndarray:
    """Locality selection at group granularity: per query partition q the
    local pair plus the n groups nearest to q, a group's distance being that
    of its closest member other than q, ties to the lower group index.

    The page selects per group (state-selection section) and motivates the
    grouping by the spatial locality of Fig. 5a; this is the fixed-policy
    counterpart of the per-pair nearest-n masks (its planner is not built).
    """
    if n < 0:
        raise ValueError("n must be >= 0")
    m = np.zeros((P, P), dtype=np.uint8)
    for q in range(P):
        m[q, q] = 1
        cands = []
        for j in range(n_groups(P, g)):
            mem = slot_members(P, g, q, 1 + j)
            if mem:
                cands.append((min(abs(q - k) for k in mem), j, mem))
        cands.sort(key=lambda c: (c[0], c[1]))
        for _, _, mem in cands[:n]:
            m[q, mem] = 1
    return m


class GroupedStateReuseOracle:
    """Selective compute and reuse with one cached state per (query partition, slot)."""

    def __init__(self, N: int, P: int, d: int, g: int, scale: float | None = None, rows=None):
        if g < 1:
            raise ValueError("group size must be >= 1")
        self.N, self.P, self.d = N, P, d
        self.g0 = self.g = g
        self.scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        self.bounds = partition_bounds(N, P)
        all_rows = np.arange(N) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
        self.part_rows = [all_rows[(all_rows >= lo) & (all_rows < hi)] for lo, hi in self.bounds]
        self.rows = all_rows
        self.reset()

    @property
    def slots(self) -> int:
        return n_slots(self.P, self.g)

    def reset(self):
        """Back to the original group size with an empty cache (before an anchor step)."""
        self.g = self.g0
        self.tc = np.full((self.P, self.slots), -1, dtype=np.int64)
        self.cache: dict = {}      # (h, q, s) -> (OUT [rows_q, d], LSE [rows_q])

    def _group_state(self, Qh, Kh, Vh, q, members):
        """Ring-based composed attention over the members, in ascending order."""
        rq = self.part_rows[q]
        st = None
        for k in members:
            lo, hi = self.bounds[k]
            part = partial_state(Qh[rq], Kh[lo:hi], Vh[lo:hi], self.scale)
            st = part if st is None else compose2(st, part)
        return st

    def step(self, t: int, mask: np.ndarray, inputs: dict):
        """Run step t with pair mask `mask`; inputs {h: (Q, K, V)} float64 [N, d].

        Returns dict with per-head merged 'O' and 'LSE' (tracked rows), the
        slot decisions 'computed' [P][slots], 'tc' [P][slots] and 'fresh'
        {(h, q, s): state}.  Raises ReuseError before touching the cache if
        a reused non-empty slot holds no state.
        """
        P = self.P
        dec = group_decisions(np.asarray(mask, dtype=np.uint8).reshape(P, P), self.g)
        for q in range(P):
            for s in range(self.slots):
                if slot_members(P, self.g, q, s) and not dec[q, s] and self.tc[q, s] < 0:
                    raise ReuseError(f"slot (q={q}, s={s}) reused at step {t} but never computed")
        outs, lses, fresh = {}, {}, {}
        for h, (Qh, Kh, Vh) in inputs.items():
            o_parts, l_parts = [], []
            for q in range(P):
                if self.part_rows[q].size == 0:
                    continue
                states = []
                for s in range(self.slots):
                    mem = slot_members(P, self.g, q, s)
                    if not mem:
                        continue
                    if dec[q, s]:
                        st = self._group_state(Qh, Kh, Vh, q, mem)
                        self.cache[(h, q, s)] = st
                        fresh[(h, q, s)] = st
                    else:
                        st = self.cache[(h, q, s)]
                    states.append(st)
                o, l = compose(states)
                o_parts.append(o)
                l_parts.append(l)
            outs[h] = np.concatenate(o_parts, axis=0)
            lses[h] = np.concatenate(l_parts, axis=0)
        self.tc[dec == 1] = t
        return {"O": outs, "LSE": lses, "fresh": fresh, "computed": dec, "tc": self.tc.copy()}

    def fit_memory(self, budget: int, k: int, bytes_per_slot: int) -> int:
        """Merge groups k at a time while the cache exceeds the budget;
        returns the number of merges (Dynamic Group State Compose)."""
        n = merges_to_fit(self.P, self.g, k, bytes_per_slot, budget)
        for _ in range(n):
            self.compose_groups(k)
        return n

    def compose_groups(self, k: int):
        """Dynamic Group State Compose: group size g -> k g, composing cached states."""
        if k < 2:
            raise ValueError("merge factor must be >= 2")
        P, g_old = self.P, self.g
        m_old, g_new = n_groups(P, g_old), k * g_old
        m_new = n_groups(P, g_new)
        heads = sorted({h for (h, _, _) in self.cache})
        tc_new = np.full((P, n_slots(P, g_new)), -1, dtype=np.int64)
        cache_new = {}
        for q in range(P):
            tc_new[q, 0] = self.tc[q, 0]
            for h in heads:
                if (h, q, 0) in self.cache:
                    cache_new[(h, q, 0)] = self.cache[(h, q, 0)]
            for i in range(m_new):
                parts = [j for j in range(k * i, min(k * i + k, m_old)) if slot_members(P, g_old, q, 1 + j)]
                if not parts:
                    continue
                if any(self.tc[q, 1 + j] < 0 for j in parts):
                    raise ReuseError(f"query partition {q}: group merge over a slot that holds no state")
                tc_new[q, 1 + i] = min(self.tc[q, 1 + j] for j in parts)
                for h in heads:
                    cache_new[(h, q, 1 + i)] = compose([self.cache[(h, q, 1 + j)] for j in parts])
        self.g, self.tc, self.cache = g_new, tc_new, cache_new
