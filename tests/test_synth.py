"""The seeded input generator: rounding, encoding and determinism (CPU only)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_positional_encoding_norm_and_blocks():
    for name in ("tiny", "image", "video_25", "stress"):
        w = synth.get(name)
        pe = synth.pos_encoding(w).astype(np.float64)
        # every (sin, cos) channel pair has squared norm A^2
        np.testing.assert_allclose((pe ** 2).sum(1), w.pe_amp ** 2 * w.d / 2, rtol=1e-5)
    w = synth.get("image")                       # one frame: the frame block is constant
    pe = synth.pos_encoding(w)
    df = w.d - 4 * (w.d // 6)
    assert np.all(pe[:, :df] == pe[0, :df])


def test_generator_deterministic_and_head_subsets_agree():
    w = synth.get("tiny")
    a = synth.step_inputs(w, 1)
    b = synth.step_inputs(w, 1, heads=[1])
    for x, y in zip(a, b):
        assert np.array_equal(x[1], y[0])
    c = synth.step_inputs(w, 1)
    assert all(np.array_equal(x, y) for x, y in zip(a, c))


def test_drift_has_stated_size():
    w = synth.get("tiny")
    m0 = synth.step_masters(w, 0)
    m1 = synth.step_masters(w, 1)
    for x0, x1 in zip(m0, m1):
        diff = (x1 - x0).astype(np.float64)
        assert abs(diff.std() - w.sigma) < 0.002
    # the encoding is on Q and K only
    pe = synth.pos_encoding(w)
    q0, k0, v0 = m0
    assert abs((q0 - pe).std() - 1) < 0.01 and abs(v0.std() - 1) < 0.01


def test_shapes():
    w = synth.get("stress")
    assert (w.N, w.S, w.N - 31 * w.S) == (17550, 549, 531)
    assert synth.get("long").N == 75600 and synth.get("video_50").N == 32760
    assert synth.get("image").N == 16384
