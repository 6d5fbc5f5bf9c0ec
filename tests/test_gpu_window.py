"""GPU parity of window attention with residual sharing (partition
granularity) against the fp64 oracle (oracle.window_residual), through the
C ABI: the full step's output, LSE and cached residual, and every window
step's output and LSE, at the per-pair bar (OUT max-abs <= 2e-2, mean-abs
<= 2e-3, LSE abs <= 1e-3; the residual is a difference of two outputs and is
held to the OUT bar)."""
import numpy as np
import pytest

import synth
from oracle.masks import nearest_mask, radius_mask
from oracle.window_residual import WindowResidualOracle

from gpu_run import log, run_window_residual_steps
from test_gpu_parity import _sample_rows, _scaled, check_state

pytestmark = pytest.mark.gpu


def _window(w):
    return radius_mask(w.P, 1) if w.policy == "radius" else nearest_mask(w.P, min(w.n_fresh, w.P))


def _compare(w, rows=None, heads=None, steps=None, label=None, state_dtype="fp32"):
    from synth import InputStream, bf16_bits_to_f64
    import torch
    steps = w.steps if steps is None else steps
    heads = list(range(w.H)) if heads is None else heads
    win = _window(w)
    orc = WindowResidualOracle(w.N, w.P, w.d, rows=rows)
    stream = InputStream(w, heads)
    ref = {}
    for t in range(steps):
        qb, kb, vb = stream.next()
        x = {h: (bf16_bits_to_f64(qb[i]), bf16_bits_to_f64(kb[i]), bf16_bits_to_f64(vb[i])) for i, h in enumerate(heads)}
        res = orc.full_step(win, x) if t == 0 else orc.window_step(win, x)
        ref[t] = (res, {h: orc.residual[h].copy() for h in heads})
    hsel = torch.tensor(heads, device="cuda")
    rws = orc.rows

    def check(t, cache, R, O, LSE):
        res, resid = ref[t]
        Oc, Lc, Rc = O[hsel].cpu().numpy(), LSE[hsel].cpu().numpy(), R[hsel].cpu().numpy()
        for i, h in enumerate(heads):
            check_state(Oc[i, rws], Lc[i, rws], res["O"][h], res["LSE"][h], f"{label} step {t} head {h}")
            if t == 0:
                check_state(Rc[i, rws], np.zeros(len(rws)), resid[h], np.zeros(len(rws)),
                            f"{label} residual head {h}")

    run_window_residual_steps(w, win, steps=steps, on_step=check, label=label, state_dtype=state_dtype)
    log(f"  {label}: ok")


CASES = [
    synth.get("tiny"),
    _scaled("image", "image_small", 1, 57, 97, 2),
    _scaled("video_25", "video25_small", 5, 21, 29, 2),
    _scaled("long", "long_small", 7, 19, 23, 2),
    _scaled("stress", "stress_small", 5, 16, 27, 2, steps=4),
    synth.get("video_100").scaled(name="p1_wr", F=1, Hh=10, W=30, H=2, P=1, steps=2, n_fresh=1),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_window_residual_matches_oracle(w):
    _compare(w, label=w.name)


@pytest.mark.parametrize("w", [CASES[1], CASES[3]], ids=[CASES[1].name, CASES[3].name])
def test_window_residual_bf16_states_match_oracle(w):
    """The window states composed from bf16 OUT; the residual stays fp32."""
    _compare(w, label=f"{w.name} bf16 states", state_dtype="bf16")


def test_window_residual_full_size_sampled_rows():
    w = synth.get("video_25")
    _compare(w, rows=_sample_rows(w), heads=[0, w.H - 1], steps=3, label="video_25 full")
