"""Selective compute and reuse of attention states across denoising steps, fp64.

DiTango page:

* selective compute and reuse (Fig. 6): at step t fresh states are computed
  for the selected KV partitions while the states of the others are taken
  from the cache instead of recomputing them;
* state selection: t_c is the last step at which a unit was computed, so a
  reused state is the one cached at t_c (not necessarily t - 1);
* anchor steps: every unit computes and t_c <- t;
* ring-based composed attention: fresh states go to the attention-state
  cache for reuse at later steps;
* composition (Eq. 4): the final output of a query row is the composition of
  its P pair states.

The unit is one (query partition q, KV partition k) pair.  ``rows`` may
restrict the oracle to a subset of query rows (sampled checks at full size);
each pair state is a function of its own query rows only, so tracking a
subset is exact for those rows.
"""
from __future__ import annotations

import numpy as np

from .state import compose, partial_state, partition_bounds
from .masks import step_mask


class ReuseError(RuntimeError):
    """A pair marked REUSE has no cached state (never computed)."""


class StateReuseOracle:
    def __init__(self, N: int, P: int, d: int, scale: float | None = None, rows=None):
        self.N, self.P, self.d = N, P, d
        self.scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        self.bounds = partition_bounds(N, P)
        all_rows = np.arange(N) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
        # tracked query rows of each partition
        self.part_rows = [all_rows[(all_rows >= lo) & (all_rows < hi)] for lo, hi in self.bounds]
        self.rows = all_rows
        self.tc = np.full((P, P), -1, dtype=np.int64)
        self.cache: dict = {}          # (h, q, k) -> (OUT [rows_q, d], LSE [rows_q])

    def step(self, t: int, mask: np.ndarray, inputs: dict):
        """Run step t.

        inputs: {h: (Q, K, V)} with float64 [N, d] arrays (bf16 values).
        Returns dict with per-head merged 'O' [len(rows), d] and 'LSE',
        'fresh' {(h, q, k): state}, 'reused' (uint8 P x P) and 'tc'.
        Raises ReuseError before touching the cache if a reused pair was never
        computed.
        """
        P = self.P
        mask = np.asarray(mask, dtype=np.uint8).reshape(P, P)
        bad = (mask == 0) & (self.tc < 0)
        if bad.any():
            q, k = map(int, np.argwhere(bad)[0])
            raise ReuseError(f"pair (q={q}, k={k}) reused at step {t} but never computed")
        outs, lses, fresh = {}, {}, {}
        for h, (Qh, Kh, Vh) in inputs.items():
            o_parts, l_parts = [], []
            for q in range(P):
                rq = self.part_rows[q]
                if rq.size == 0:
                    continue
                states = []
                for k in range(P):
                    klo, khi = self.bounds[k]
                    if mask[q, k]:
                        st = partial_state(Qh[rq], Kh[klo:khi], Vh[klo:khi], self.scale)
                        self.cache[(h, q, k)] = st
                        fresh[(h, q, k)] = st
                    else:
                        st = self.cache[(h, q, k)]
                    states.append(st)
                o, l = compose(states)
                o_parts.append(o)
                l_parts.append(l)
            outs[h] = np.concatenate(o_parts, axis=0)
            lses[h] = np.concatenate(l_parts, axis=0)
        self.tc[mask == 1] = t
        return {"O": outs, "LSE": lses, "fresh": fresh,
                "reused": (mask == 0).astype(np.uint8), "tc": self.tc.copy()}


def run_workload(w, heads=None, rows=None, steps=None, masks=None, on_step=None, fp32_masters=False):
    """Run the oracle over the steps of workload w (synthetic inputs from synth).

    masks: optional {t: mask} overriding the workload's policy.
    fp32_masters: feed the unrounded fp32 master tensors instead of their bf16
    copies (for workloads specified in fp32).
    on_step(t, mask, result) is called after each step; returns the last result.
    """
    from synth import InputStream, bf16_bits_to_f64  # the shared seeded generator

    heads = list(range(w.H)) if heads is None else list(heads)
    n_steps = w.steps if steps is None else steps
    orc = StateReuseOracle(w.N, w.P, w.d, rows=rows)
    stream = InputStream(w, heads)
    res = None
    for t in range(n_steps):
        qb, kb, vb = stream.next()
        mask = step_mask(w, t) if masks is None or t not in masks else masks[t]
        if fp32_masters:
            inputs = {h: tuple(m[i].astype(np.float64) for m in stream.masters) for i, h in enumerate(heads)}
        else:
            inputs = {h: (bf16_bits_to_f64(qb[i]), bf16_bits_to_f64(kb[i]), bf16_bits_to_f64(vb[i]))
                      for i, h in enumerate(heads)}
        res = orc.step(t, mask, inputs)
        if on_step is not None:
            on_step(t, mask, res)
    return res
