"""The library's own step driver (ditango_step) against the three-call
sequence it stands for: identical outputs, cache slots, t_c and reused sets,
bit for bit, over a workload with reuse."""
import numpy as np
import pytest

import synth

from gpu_run import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "image_small"])
def test_step_driver_equals_three_calls(name):
    import torch
    import context_state_reuse_amd as lib
    w = synth.get("tiny") if name == "tiny" else synth.get("image").scaled(name="image_small", F=1, Hh=57, W=97, H=2)
    a = lib.StateCache(w.H, w.N, w.d, w.P)
    b = lib.StateCache(w.H, w.N, w.d, w.P)
    stream = synth.InputStream(w)
    for t in range(w.steps):
        Q, K, V = (to_device(x) for x in stream.next())
        mask = lib.workload_mask(w, t)
        lib.ditango_attn_partial(Q, K, V, mask, a)
        ra = lib.ditango_state_cache_update(a, mask, t)
        Oa, La = lib.ditango_state_merge(a)
        Ob, Lb, rb = lib.ditango_step(Q, K, V, mask, t, b)
        torch.cuda.synchronize()
        assert np.array_equal(ra, rb) and np.array_equal(a.tc, b.tc)
        assert torch.equal(Oa, Ob) and torch.equal(La, Lb)
        for q in range(w.P):                      # rows past a ragged partition are never written
            n = min(w.S, w.N - q * w.S)
            sl = slice(q * w.P, (q + 1) * w.P)
            assert torch.equal(a.O[:, sl, :n], b.O[:, sl, :n]) and torch.equal(a.LSE[:, sl, :n], b.LSE[:, sl, :n])
