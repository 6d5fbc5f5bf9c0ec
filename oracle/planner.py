"""Anchor-guided selection of the states to compute or reuse, fp64 (test
infrastructure only).

DiTango page, error-analysis and state-selection sections (Eq. 5 to 9 and
Algorithm 1, whose display equations and listing body are lost in
extraction).  What the prose fixes:

* normalised weights w_i = exp(LSE_i) / sum_j exp(LSE_j) measure how much a
  partition's state contributes to a row's composed output; dropping the
  second-order cross term of Eq. 5 leaves (Eq. 6) the output error as the
  w-weighted sum of the states' output errors;
* the Attention State Error of a cached state is w(i, t) * delta(i, t, t_c):
  importance times an error that grows with the cache age t - t_c;
* states are grouped, the local state is handled on its own and is always
  computed; a group's ASE is the sum of its members'; the group is computed
  when its ASE exceeds a threshold eps, reused otherwise;
* anchor steps compute everything; one is triggered when the local state's
  relative error (its drift) exceeds a bound; at an anchor the importance
  weights w and the scale ratios alpha are re-measured and the compute
  steps t_c reset; eps follows a percentile of the errors corrected at the
  anchor, chosen to meet a target acceleration.

Readings where the page is silent (each the plainest one the rest
supports; parity unpinned against the page for the decision rule itself):

* importance of pair (q, k): w(q, k) = mean over the rows r of q of
  exp(LSE_qk[r] - LSE_q[r]) (the normalised weight, averaged over rows and,
  for the decision, over heads) -- the share of q's attention mass on k;
* a state's error is measured on its signature, the mean of its OUT rows
  (per head, d values): drift(new, ref) = ||new - ref|| / ||ref|| over the
  heads' signatures concatenated;
* the local drift D(q, t) is the drift of q's local signature at step t
  against its value at the last anchor; an anchor is taken at the first
  `warmup` steps (at least two: the first has nothing to correct) and
  whenever max_q D(q, t) > drift_max;
* at an anchor with a previous cache, the correction error of pair (q, k)
  is e(q, k) = drift(signature now, signature cached before the step) and
  its scale ratio alpha(q, k) = e(q, k) / D(q, t) (0 when D is 0): how fast
  the pair drifts relative to the local state;
* between anchors the predicted error of member k of group G is
  alpha(q, k) * max(0, D(q, t) - D(q, t_c(G))), where D(q, t_c(G)) is the
  local drift recorded when G was last computed (0 right after an anchor);
  ASE(q, G) = sum_k w(q, k) * that (0 when D has not grown, and a member of
  zero importance adds nothing, even with an infinite alpha);
* groups are those of the grouped cache: G_j = {j g .. min((j+1) g, P) - 1}
  minus q; a group with no member is skipped;
* eps: the errors corrected at the anchor are E(q, G) = sum_k w(q, k) e(q, k)
  over all groups with members (a member of zero importance adds nothing,
  even when its drift is +inf: its state has no weight in the output); with the target reuse fraction rho (the
  share of groups reused, which sets the acceleration), eps is the
  ceil(rho n)-th smallest of the n values (-inf when that is 0), and a
  group is reused when ASE <= eps.
"""
from __future__ import annotations

import math

import numpy as np


def pair_weights(slot_lse: np.ndarray, merged_lse: np.ndarray) -> np.ndarray:
    """Importance of every pair of one head: W[q][k] = mean_r exp(LSE_qk[r] - LSE_q[r]).

    slot_lse: [P][P][rows_q] per query partition q (a list of arrays is
    accepted for ragged partitions); merged_lse: [P][rows_q] likewise.
    """
    P = len(slot_lse)
    W = np.zeros((P, P))
    for q in range(P):
        lq = np.asarray(merged_lse[q], dtype=np.float64)
        for k in range(P):
            W[q, k] = np.mean(np.exp(np.asarray(slot_lse[q][k], dtype=np.float64) - lq))
    return W


def pair_signature(out_rows: np.ndarray) -> np.ndarray:
    """Signature of one pair state of one head: the mean of its OUT rows [rows][d] -> [d]."""
    return np.mean(np.asarray(out_rows, dtype=np.float64), axis=0)


def rel_drift(new: np.ndarray, ref: np.ndarray) -> float:
    """||new - ref|| / ||ref|| (0 when both are 0, inf when only ref is)."""
    new = np.asarray(new, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    num = math.sqrt(float(np.sum((new - ref) ** 2)))
    den = math.sqrt(float(np.sum(ref * ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def reuse_threshold(values, rho: float) -> float:
    """eps such that a fraction rho of `values` is <= eps: the ceil(rho n)-th smallest."""
    v = sorted(float(x) for x in values)
    if not v:
        return math.inf
    k = math.ceil(rho * len(v) - 1e-12)
    if k <= 0:
        return -math.inf
    return v[min(k, len(v)) - 1]


def group_members(P: int, g: int, q: int, j: int) -> list[int]:
    return [k for k in range(j * g, min((j + 1) * g, P)) if k != q]


class AnchorPlanner:
    """Per-step mask from the error model above.

    Per step t: plan(t, sig_local) with the signatures of the freshly
    computed local states gives the mask (1 = compute); after the step,
    update(t, mask, W, sig_new, sig_old) with the importance of every pair
    (merged LSE of step t), the signatures of every pair after the step and
    those cached before it (None at the first step).
    Signature arrays are [H][P][P][d] (only the diagonal of sig_local is read).
    """

    def __init__(self, P: int, g: int, target_reuse: float, drift_max: float, warmup: int = 2):
        if not (1 <= g <= P) or not (0.0 <= target_reuse <= 1.0) or warmup < 2 or not drift_max >= 0:
            raise ValueError("bad planner parameters")
        self.P, self.g = P, g
        self.m = -(-P // g)
        self.rho, self.drift_max, self.warmup = float(target_reuse), float(drift_max), warmup
        self.W = np.zeros((P, P))
        self.alpha = np.zeros((P, P))
        self.Dc = np.zeros((P, self.m))
        self.D = np.zeros(P)
        self.eps = math.inf
        self.sigref = None            # [H][P][d] local signatures at the last anchor
        self.anchor = False
        self.n_anchors = 0

    def plan(self, t: int, sig_local) -> tuple[np.ndarray, bool]:
        P = self.P
        sig = np.asarray(sig_local, dtype=np.float64)
        if self.sigref is not None:
            D = np.array([rel_drift(sig[:, q, q, :], self.sigref[:, q, :]) for q in range(P)])
        else:
            D = np.zeros(P)
        return self.plan_drift(t, D)

    def plan_drift(self, t: int, D) -> tuple[np.ndarray, bool]:
        """plan() from the local drifts D[q] themselves (ignored before the first anchor)."""
        P = self.P
        self.D = np.asarray(D, dtype=np.float64).copy() if self.n_anchors else np.zeros(P)
        self.anchor = t < self.warmup or self.n_anchors == 0 or not float(np.max(self.D)) <= self.drift_max
        if self.anchor:
            return np.ones((P, P), dtype=np.uint8), True
        ase = self.predicted_errors()
        mask = np.eye(P, dtype=np.uint8)
        for q in range(P):
            for j in range(self.m):
                mem = group_members(P, self.g, q, j)
                if mem and ase[q, j] > self.eps:
                    mask[q, mem] = 1
        return mask, False

    def predicted_errors(self) -> np.ndarray:
        """ASE of every group [P][m] from the current local drifts (NaN for a
        group without members): importance times the scale ratio times the
        local drift's growth since the group was last computed."""
        P = self.P
        ase = np.full((P, self.m), np.nan)
        for q in range(P):
            for j in range(self.m):
                mem = group_members(P, self.g, q, j)
                if not mem:
                    continue
                grow = max(0.0, self.D[q] - self.Dc[q, j])
                # no growth predicts no error; a member of zero importance adds
                # none (also when its scale ratio is +inf)
                ase[q, j] = sum(self.W[q, k] * self.alpha[q, k] * grow for k in mem if self.W[q, k] > 0) \
                    if grow > 0 else 0.0
        return ase

    def update(self, t: int, mask, W_heads, sig_new, sig_old=None) -> None:
        P = self.P
        e = None
        if self.anchor:
            sig_new = np.asarray(sig_new, dtype=np.float64)
            if sig_old is not None and self.sigref is not None:
                sig_old = np.asarray(sig_old, dtype=np.float64)
                e = np.array([[rel_drift(sig_new[:, q, k, :], sig_old[:, q, k, :]) if k != q else 0.0
                               for k in range(P)] for q in range(P)])
            self.sigref = np.array([sig_new[:, q, q, :] for q in range(P)]).transpose(1, 0, 2).copy()
        self.update_drift(t, mask, None if W_heads is None else np.mean(np.asarray(W_heads, np.float64), axis=0), e)

    def update_drift(self, t: int, mask, W, e) -> None:
        """update() from the head-mean importance W[q][k] and the pairs' drifts
        e[q][k] against the cache before the step (both read at anchors only;
        e None at the first anchor)."""
        P = self.P
        mask = np.asarray(mask, dtype=np.uint8)
        if self.anchor:
            W = np.asarray(W, dtype=np.float64)
            if not (np.all(np.isfinite(W)) and np.all(W >= 0)):
                raise ValueError("importance must be finite and >= 0")
            if e is not None and self.n_anchors > 0:
                off = ~np.eye(P, dtype=bool)
                if not np.all(np.asarray(e, dtype=np.float64)[off] >= 0):   # NaN fails too; +inf is a drift
                    raise ValueError("pair drifts must be >= 0")
            self.W = W.copy()
            if e is not None and self.n_anchors > 0:
                e = np.asarray(e, dtype=np.float64)
                for q in range(P):
                    for k in range(P):
                        if k != q:
                            self.alpha[q, k] = e[q, k] / self.D[q] if self.D[q] > 0 else 0.0
                # Eq. 6 weights each state's error by its importance: a pair of
                # zero importance adds nothing, even with an unbounded drift
                E = [sum(self.W[q, k] * e[q, k] for k in group_members(P, self.g, q, j) if self.W[q, k] > 0)
                     for q in range(P) for j in range(self.m) if group_members(P, self.g, q, j)]
                self.eps = reuse_threshold(E, self.rho)
            self.Dc[:] = 0.0
            self.n_anchors += 1
        else:
            for q in range(P):
                for j in range(self.m):
                    mem = group_members(P, self.g, q, j)
                    if mem and all(mask[q, k] for k in mem):
                        self.Dc[q, j] = self.D[q]
