"""Seeded synthetic Q/K/V for the DiT-shaped workloads.

Recipe (the pages give no data; their workloads are Wan2.1 / PixArt-Sigma
latents, which these tensors stand in for):

* step 0: Q, K, V ~ N(0, 1) per element, and a 3D sinusoidal positional
  encoding of amplitude ``pe_amp`` added to Q and K (not V), so that
  attention mass concentrates on spatially near tokens -- the locality DiTango
  measures in its partition-importance study (Fig. 5a of the DiTango page).
* step t >= 1: each fp32 master tensor drifts, X_t = X_{t-1} + sigma * eps_t,
  with fresh independent noise eps_t; the encoding is not re-added.
* both the GPU path and the oracle consume the same bf16 (round to nearest
  even) copy of the fp32 master of each step.

Noise streams are NumPy ``default_rng(SeedSequence([cfg_id, t, tensor, h]))``
with tensor Q=0, K=1, V=2, one (N, d) float32 draw per head, so any subset of
heads can be regenerated on its own.

Positional encoding: the head dimension is split into [frame | row | column]
blocks with d_row = d_col = 2*floor(d/6) and d_frame = d - d_row - d_col; in a
block of even width m for coordinate c, channel 2i holds A*sin(c*10000^(-2i/m))
and channel 2i+1 holds A*cos(c*10000^(-2i/m)).

This module holds no arithmetic of the attention method itself.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

Q_ID, K_ID, V_ID = 0, 1, 2


def token_coords(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(frame, row, col) of every token in frame-major order."""
    n = np.arange(w.N, dtype=np.int64)
    return n // (w.Hh * w.W), (n // w.W) % w.Hh, n % w.W


def pos_encoding(w: Workload) -> np.ndarray:
    """[N, d] float32 3D sinusoidal encoding (same for every head)."""
    d = w.d
    dy = dx = 2 * (d // 6)
    df = d - dy - dx
    f, y, x = token_coords(w)
    pe = np.zeros((w.N, d), dtype=np.float64)
    off = 0
    for coord, m in ((f, df), (y, dy), (x, dx)):
        half = m // 2
        freq = 10000.0 ** (-2.0 * np.arange(half) / m)
        ang = coord[:, None].astype(np.float64) * freq[None, :]
        pe[:, off:off + m:2] = w.pe_amp * np.sin(ang)
        pe[:, off + 1:off + m:2] = w.pe_amp * np.cos(ang)
        off += m
    return pe.astype(np.float32)


def _noise(w: Workload, t: int, tensor: int, h: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([w.cfg_id, t, tensor, h]))
    return rng.standard_normal((w.N, w.d), dtype=np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


class InputStream:
    """Iterates the denoising steps of one workload for a subset of heads.

    ``next()`` returns (q, k, v) for the following step as bf16 bit patterns
    (uint16, shape [len(heads), N, d]); ``masters`` holds the fp32 tensors.
    """

    def __init__(self, w: Workload, heads=None):
        self.w = w
        self.heads = list(range(w.H)) if heads is None else list(heads)
        self.t = -1
        self.masters: list[np.ndarray] | None = None
        self._pe = None

    def _init_masters(self):
        w = self.w
        self._pe = pos_encoding(w)
        self.masters = []
        for tensor in (Q_ID, K_ID, V_ID):
            m = np.empty((len(self.heads), w.N, w.d), dtype=np.float32)
            for i, h in enumerate(self.heads):
                m[i] = _noise(w, 0, tensor, h)
                if tensor != V_ID:
                    m[i] += self._pe
            self.masters.append(m)

    def advance(self):
        """Move the fp32 masters to the next step."""
        self.t += 1
        if self.t == 0:
            self._init_masters()
            return
        s = np.float32(self.w.sigma)
        for tensor, m in zip((Q_ID, K_ID, V_ID), self.masters):
            for i, h in enumerate(self.heads):
                m[i] += s * _noise(self.w, self.t, tensor, h)

    def bf16(self):
        return tuple(to_bf16_bits(m) for m in self.masters)

    def next(self):
        self.advance()
        return self.bf16()


def step_inputs(w: Workload, t: int, heads=None):
    """bf16 bit patterns (q, k, v) of step t, regenerated from scratch."""
    s = InputStream(w, heads)
    for _ in range(t + 1):
        s.advance()
    return s.bf16()


def step_masters(w: Workload, t: int, heads=None):
    """fp32 masters (q, k, v) of step t (before bf16 rounding)."""
    s = InputStream(w, heads)
    for _ in range(t + 1):
        s.advance()
    return tuple(m.copy() for m in s.masters)
