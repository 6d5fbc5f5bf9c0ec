"""Window attention with residual sharing at partition granularity, fp64
(test infrastructure only).

DiTFastAttn page (approach; the techniques of its ablation table): window
attention plus a cached residual -- at a step that computes full attention,
the difference between the full output and the window output is cached; at
later steps only the window is computed and the cached residual is added to
its output.  The page gives no equations; the plainest reading at the
granularity of this library (states per (query partition, KV partition)
pair, composed with the DiTango page's Eq. 4):

* the window of query partition q is the set of KV partitions k with
  window_mask[q][k] = 1 (the near partitions, like the per-pair masks);
* full step: every pair state is computed; OUT_full and LSE_full are the
  composition of all P states of a row, OUT_win the composition of the
  window states, and the residual R = OUT_full - OUT_win is cached (output
  only -- the page caches outputs, not log-sum-exps);
* window step: only the window pairs are computed; OUT = OUT_win + R, and the
  LSE reported is the window composition's.
"""
from __future__ import annotations

import numpy as np

from .state import compose, partial_state, partition_bounds


class WindowResidualOracle:
    def __init__(self, N: int, P: int, d: int, scale: float | None = None, rows=None):
        self.N, self.P, self.d = N, P, d
        self.scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
        self.bounds = partition_bounds(N, P)
        all_rows = np.arange(N) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
        self.part_rows = [all_rows[(all_rows >= lo) & (all_rows < hi)] for lo, hi in self.bounds]
        self.rows = all_rows
        self.residual: dict = {}     # h -> R [tracked rows, d]

    def _states(self, Qh, Kh, Vh, q, ks):
        rq = self.part_rows[q]
        return [partial_state(Qh[rq], Kh[lo:hi], Vh[lo:hi], self.scale)
                for lo, hi in (self.bounds[k] for k in ks)]

    def _check_window(self, window_mask):
        w = np.asarray(window_mask, dtype=np.uint8).reshape(self.P, self.P)
        if not all(w[q].any() for q in range(self.P)):
            raise ValueError("every query partition needs at least one window partition")
        return w

    def full_step(self, window_mask, inputs: dict):
        """All pairs fresh; returns {'O', 'LSE'} of full attention and caches R."""
        w = self._check_window(window_mask)
        outs, lses = {}, {}
        for h, (Qh, Kh, Vh) in inputs.items():
            o_parts, l_parts, r_parts = [], [], []
            for q in range(self.P):
                if self.part_rows[q].size == 0:
                    continue
                st = self._states(Qh, Kh, Vh, q, range(self.P))
                o_full, l_full = compose(st)
                o_win, _ = compose([st[k] for k in range(self.P) if w[q, k]])
                o_parts.append(o_full)
                l_parts.append(l_full)
                r_parts.append(o_full - o_win)
            outs[h] = np.concatenate(o_parts, axis=0)
            lses[h] = np.concatenate(l_parts, axis=0)
            self.residual[h] = np.concatenate(r_parts, axis=0)
        return {"O": outs, "LSE": lses}

    def window_step(self, window_mask, inputs: dict):
        """Window pairs fresh; returns {'O' = OUT_win + R, 'LSE' = LSE_win}."""
        w = self._check_window(window_mask)
        outs, lses = {}, {}
        for h, (Qh, Kh, Vh) in inputs.items():
            if h not in self.residual:
                raise RuntimeError(f"head {h}: window step before any full step")
            o_parts, l_parts = [], []
            for q in range(self.P):
                if self.part_rows[q].size == 0:
                    continue
                ks = [k for k in range(self.P) if w[q, k]]
                o_win, l_win = compose(self._states(Qh, Kh, Vh, q, ks))
                o_parts.append(o_win)
                l_parts.append(l_win)
            outs[h] = np.concatenate(o_parts, axis=0) + self.residual[h]
            lses[h] = np.concatenate(l_parts, axis=0)
        return {"O": outs, "LSE": lses}
