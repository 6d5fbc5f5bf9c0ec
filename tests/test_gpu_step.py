"""The fused step launch against the three calls it stands for.

ditango_step (one fused partial + composition launch, then the t_c update)
against ditango_attn_partial, ditango_state_cache_update and
ditango_state_merge called one by one: the same reused sets and t_c, cache
slots bit for bit (the fresh states come from the same per-pair arithmetic),
the composed output equal up to the rounding of the composition's sums
(the two kernels sum the P weights in different orders).  The oracle parity
of the fused path itself is checked with the other parity workloads."""
import numpy as np
import pytest

import synth

from gpu_run import to_device

pytestmark = pytest.mark.gpu

REL_O, ABS_LSE = 1e-5, 1e-5


def _compare_paths(w, masks=None, state_dtype="fp32"):
    import torch
    import context_state_reuse_amd as lib
    a = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=state_dtype)
    b = lib.StateCache(w.H, w.N, w.d, w.P, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    for t in range(w.steps):
        Q, K, V = (to_device(x) for x in stream.next())
        mask = lib.workload_mask(w, t) if masks is None or t not in masks else np.asarray(masks[t], np.uint8)
        lib.ditango_attn_partial(Q, K, V, mask, a)
        ra = lib.ditango_state_cache_update(a, mask, t)
        Oa, La = lib.ditango_state_merge(a)
        Ob, Lb, rb = lib.ditango_step(Q, K, V, mask, t, b)
        torch.cuda.synchronize()
        assert np.array_equal(ra, rb) and np.array_equal(a.tc, b.tc)
        assert torch.isfinite(Ob).all() and torch.isfinite(Lb).all()
        rel = ((Oa - Ob).abs().max() / Oa.abs().max()).item()
        assert rel <= REL_O, f"step {t}: fused output differs by {rel:.3g} of max |O|"
        assert (La - Lb).abs().max().item() <= ABS_LSE * max(1.0, La.abs().max().item())
        for q in range(w.P):                      # rows past a ragged partition are never written
            n = min(w.S, w.N - q * w.S)
            sl = slice(q * w.P, (q + 1) * w.P)
            assert torch.equal(a.O[:, sl, :n], b.O[:, sl, :n]) and torch.equal(a.LSE[:, sl, :n], b.LSE[:, sl, :n])


SMALL = {"tiny": lambda: synth.get("tiny"),
         "image_small": lambda: synth.get("image").scaled(name="image_small", F=1, Hh=57, W=97, H=2),
         "long_small": lambda: synth.get("long").scaled(name="long_small", F=7, Hh=19, W=23, H=2),
         "stress_small": lambda: synth.get("stress").scaled(name="stress_small", F=5, Hh=16, W=27, H=3)}


@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("name", ["tiny", "image_small", "long_small", "stress_small"])
def test_fused_step_equals_three_calls(name, state_dtype):
    _compare_paths(SMALL[name](), state_dtype=state_dtype)


def test_fused_rows_without_fresh_pairs():
    """Steps where some or all query partitions compute nothing (rows of the
    mask all REUSE) and a single partition."""
    w = synth.get("video_50").scaled(name="nf0", F=3, Hh=12, W=19, H=2, steps=4)
    P = w.P
    m1 = np.zeros((P, P), np.uint8)
    m1[0, :] = 1
    m1[P - 1, P - 1] = 1
    _compare_paths(w, masks={1: m1, 2: np.zeros((P, P), np.uint8)})
    _compare_paths(synth.get("video_100").scaled(name="p1", F=1, Hh=10, W=30, H=2, P=1, steps=2, n_fresh=1))


def test_partial_merge_leaves_tc_and_checks_cache():
    import torch
    import context_state_reuse_amd as lib
    w = synth.get("video_50").scaled(name="pm", F=2, Hh=9, W=17, H=2, steps=2)
    cache = lib.StateCache(w.H, w.N, w.d, w.P)
    Q, K, V = (to_device(x) for x in synth.InputStream(w).next())
    with pytest.raises(lib.DitangoError) as e:           # REUSE pairs with no state: no launch
        lib.ditango_attn_partial_merge(Q, K, V, lib.ditango_mask_build("nearest", w.P, 2), cache)
    assert e.value.code == lib.DITANGO_ENOCACHE
    ones = np.ones((w.P, w.P), np.uint8)
    O1, L1 = lib.ditango_attn_partial_merge(Q, K, V, ones, cache)
    assert (cache.tc < 0).all()
    O2, L2, _ = lib.ditango_step(Q, K, V, ones, 0, cache)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert (cache.tc == 0).all()


GROUP_CASES = [("stress_small", 4, "fp32"), ("image_small", 3, "fp32"), ("long_small", 4, "fp32"),
               ("stress_small", 4, "bf16"), ("long_small", 4, "bf16")]


@pytest.mark.parametrize("name,g,state_dtype", GROUP_CASES, ids=[f"{n}_g{g}_{s}" for n, g, s in GROUP_CASES])
def test_group_fused_step_equals_two_launches(name, g, state_dtype):
    """The grouped cache: ditango_group_attn_partial_merge against
    ditango_group_attn_partial + ditango_group_merge -- slot states bit for
    bit, the composed output within fp32 rounding of the weight sums."""
    import torch
    import context_state_reuse_amd as lib
    w = SMALL[name]()
    a = lib.GroupedStateCache(w.H, w.N, w.d, w.P, g, state_dtype=state_dtype)
    b = lib.GroupedStateCache(w.H, w.N, w.d, w.P, g, state_dtype=state_dtype)
    stream = synth.InputStream(w)
    for t in range(w.steps):
        Q, K, V = (to_device(x) for x in stream.next())
        mask = lib.workload_mask(w, t)
        lib.ditango_group_attn_partial(Q, K, V, mask, a)
        ca = lib.ditango_group_cache_update(a, mask, t)
        Oa, La = lib.ditango_group_merge(a)
        Ob, Lb = lib.ditango_group_attn_partial_merge(Q, K, V, mask, b)
        cb = lib.ditango_group_cache_update(b, mask, t)
        torch.cuda.synchronize()
        assert np.array_equal(ca, cb) and np.array_equal(a.tc, b.tc)
        rel = ((Oa - Ob).abs().max() / Oa.abs().max()).item()
        assert rel <= REL_O, f"step {t}: fused output differs by {rel:.3g} of max |O|"
        assert (La - Lb).abs().max().item() <= ABS_LSE * max(1.0, La.abs().max().item())
        for s in range(a.n_slots):
            for q in range(w.P):
                if not lib.group_slot_live(w.P, g, q, s):
                    continue
                n = min(w.S, w.N - q * w.S)
                assert torch.equal(a.O[s][:, q, :n], b.O[s][:, q, :n]) and torch.equal(a.LSE[s][:, q, :n], b.LSE[s][:, q, :n])
