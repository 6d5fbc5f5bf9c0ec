"""Pins of the oracle's attention state and composition (CPU only).

Each test checks the oracle against something other than itself: brute-force
softmax attention written with scalar loops, torch's own attention routine,
closed forms, and the composition laws the DiTango page states (composition
is associative and commutative; Eq. 4; the ring of g partial steps yields the
whole group state).
"""
import math

import numpy as np
import pytest
import torch

from oracle.state import compose, compose2, partial_state, partition_bounds
from oracle.reuse import StateReuseOracle


def brute_attention(q, k, v, scale):
    """Full softmax attention with Python scalars: (out [rows, d], lse [rows])."""
    rows, d = q.shape
    nk = k.shape[0]
    out = np.zeros((rows, v.shape[1]))
    lse = np.zeros(rows)
    for i in range(rows):
        z = [scale * sum(float(q[i, c]) * float(k[j, c]) for c in range(d)) for j in range(nk)]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        den = sum(e)
        lse[i] = m + math.log(den)
        for j in range(nk):
            out[i] += (e[j] / den) * v[j]
    return out, lse


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_partition_bounds_ragged_and_errors():
    assert partition_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert partition_bounds(1024, 4) == [(0, 256), (256, 512), (512, 768), (768, 1024)]
    b = partition_bounds(17550, 32)
    assert b[0] == (0, 549) and b[-1] == (31 * 549, 17550) and b[-1][1] - b[-1][0] == 531
    with pytest.raises(ValueError):
        partition_bounds(10, 6)        # S = 2 -> partition 5 would be empty
    with pytest.raises(ValueError):
        partition_bounds(0, 1)


@pytest.mark.parametrize("N,P,d", [(13, 1, 4), (13, 3, 4), (23, 5, 3), (31, 7, 5), (16, 4, 8)])
def test_all_fresh_equals_brute_force(N, P, d):
    """With every pair fresh, composing the P pair states is full attention."""
    q, k, v = rand((N, d), 1, 1.5), rand((N, d), 2, 1.5), rand((N, d), 3)
    scale = 1 / math.sqrt(d)
    orc = StateReuseOracle(N, P, d)
    res = orc.step(0, np.ones((P, P), np.uint8), {0: (q, k, v)})
    ob, lb = brute_attention(q, k, v, scale)
    np.testing.assert_allclose(res["O"][0], ob, atol=1e-12, rtol=0)
    np.testing.assert_allclose(res["LSE"][0], lb, atol=1e-12, rtol=0)


@pytest.mark.parametrize("N,P", [(300, 1), (300, 7), (257, 2), (100, 5)])
def test_all_fresh_equals_torch_sdpa(N, P):
    """Cross-check with torch's attention routine (fp64, CPU) and logsumexp."""
    d = 16
    q, k, v = rand((N, d), 4, 2.0), rand((N, d), 5, 2.0), rand((N, d), 6)
    orc = StateReuseOracle(N, P, d)
    res = orc.step(0, np.ones((P, P), np.uint8), {0: (q, k, v)})
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    ref_lse = torch.logsumexp(torch.from_numpy(q @ k.T) / math.sqrt(d), dim=1).numpy()
    np.testing.assert_allclose(res["O"][0], ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(res["LSE"][0], ref_lse, atol=1e-12, rtol=0)


def test_closed_form_zero_keys():
    """K = 0: every score is 0, so OUT is the mean of V and LSE = log(#keys)."""
    q, v = rand((6, 5), 7), rand((9, 5), 8)
    o, l = partial_state(q, np.zeros((9, 5)), v, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-15)
    np.testing.assert_allclose(l, np.full(6, math.log(9)), atol=1e-15)


def test_closed_form_single_key():
    """One key: OUT = v and LSE = s * q.k."""
    q, k, v = rand((4, 6), 9), rand((1, 6), 10), rand((1, 6), 11)
    o, l = partial_state(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-15)
    np.testing.assert_allclose(l, 0.25 * (q @ k[0]), atol=1e-14)


def test_score_shift_moves_lse_only():
    """Adding c to every score of a row leaves OUT unchanged and adds c to LSE."""
    d, s, c = 8, 0.4, 3.7
    q, k, v = rand((1, d), 12), rand((11, d), 13), rand((11, d), 14)
    u = q[0] * (c / (s * float(q[0] @ q[0])))       # q.u = c / s for the single row
    o1, l1 = partial_state(q, k, v, s)
    o2, l2 = partial_state(q, k + u, v, s)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-12)


def test_lse_is_log_of_softmax_denominator():
    """exp(LSE) equals the plain sum of exp(scores) on a small well-scaled case."""
    q, k, v = rand((3, 4), 15, 0.5), rand((7, 4), 16, 0.5), rand((7, 4), 17)
    _, l = partial_state(q, k, v, 0.5)
    np.testing.assert_allclose(np.exp(l), np.exp(0.5 * (q @ k.T)).sum(1), rtol=1e-14)


def _states(n, rows=5, d=4, seed=20):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((rows, d)), rng.standard_normal(rows) * 5) for _ in range(n)]


def test_compose_commutative():
    st = _states(7)
    o, l = compose(st)
    rng = np.random.default_rng(1)
    for _ in range(5):
        perm = rng.permutation(len(st))
        o2, l2 = compose([st[i] for i in perm])
        np.testing.assert_allclose(o2, o, atol=1e-13)
        np.testing.assert_allclose(l2, l, atol=1e-13)


def test_compose_associative_random_trees():
    """Any binary tree of pairwise compositions (Eq. 4) equals the n-ary merge."""
    st = _states(9, seed=21)
    o, l = compose(st)
    rng = np.random.default_rng(2)
    for _ in range(10):
        pool = list(st)
        while len(pool) > 1:
            i, j = sorted(rng.choice(len(pool), 2, replace=False))
            b = pool.pop(j)
            a = pool.pop(i)
            pool.append(compose2(a, b))
        np.testing.assert_allclose(pool[0][0], o, atol=1e-13)
        np.testing.assert_allclose(pool[0][1], l, atol=1e-13)


def test_compose_of_disjoint_key_sets_is_union_state():
    """Eq. 4 on real states: the states of two key sets compose to the union's state."""
    q, k, v = rand((6, 5), 30), rand((20, 5), 31), rand((20, 5), 32)
    s = 0.7
    whole = partial_state(q, k, v, s)
    sel = np.random.default_rng(3).permutation(20)
    a, b = sel[:8], sel[8:]
    u = compose2(partial_state(q, k[a], v[a], s), partial_state(q, k[b], v[b], s))
    np.testing.assert_allclose(u[0], whole[0], atol=1e-13)
    np.testing.assert_allclose(u[1], whole[1], atol=1e-13)


@pytest.mark.parametrize("g", [2, 3, 5])
def test_ring_of_sub_blocks_equals_whole_partition(g):
    """Ring-based composed attention: g partial steps folded in one by one give
    the state of the whole group (DiTango page, ring-based composed attention)."""
    q, k, v = rand((4, 6), 40, 2), rand((23, 6), 41, 2), rand((23, 6), 42)
    s = 1 / math.sqrt(6)
    whole = partial_state(q, k, v, s)
    blocks = np.array_split(np.arange(23), g)
    acc = partial_state(q, k[blocks[0]], v[blocks[0]], s)
    for b in blocks[1:]:
        acc = compose2(acc, partial_state(q, k[b], v[b], s))
    np.testing.assert_allclose(acc[0], whole[0], atol=1e-13)
    np.testing.assert_allclose(acc[1], whole[1], atol=1e-13)


def test_first_order_error_propagation_weights():
    """Error analysis (Eq. 5/6): an error dOUT_i in one state reaches the merged
    output scaled by its normalised weight w_i = exp(LSE_i - LSE); an error in
    LSE_i moves the output by w_i * dLSE_i * (OUT_i - OUT) to first order."""
    st = _states(4, rows=3, d=5, seed=50)
    o, l = compose(st)
    w = [np.exp(s[1] - l) for s in st]
    np.testing.assert_allclose(sum(w), np.ones(3), atol=1e-14)
    delta = np.random.default_rng(4).standard_normal((3, 5)) * 1e-3
    i = 2
    pert = list(st)
    pert[i] = (st[i][0] + delta, st[i][1])
    o2, _ = compose(pert)
    np.testing.assert_allclose(o2 - o, w[i][:, None] * delta, atol=1e-15)
    eps = 1e-6
    pert = list(st)
    pert[i] = (st[i][0], st[i][1] + eps)
    o3, _ = compose(pert)
    pred = w[i][:, None] * eps * (st[i][0] - o)
    np.testing.assert_allclose(o3 - o, pred, atol=1e-11)
