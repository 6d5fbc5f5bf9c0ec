"""Workload shapes for partitioned attention with selective state reuse.

Each workload is a DiT attention layer over a 3D latent (frames x height x
width) flattened frame-major into one token sequence, as DiTango's
introduction describes for 3D full attention.  The sequence is cut into P
contiguous context-parallel partitions (the Ring-CP sequence partitioning
of the same page), and every denoising step t >= 1 runs with a per-step
selection mask over the P x P (query partition, KV partition) pairs.  Step 0
is an anchor step (all pairs fresh), as the page's anchor-step section
prescribes.

This module holds shapes and knobs only; it holds none of the method's
arithmetic.  The mask *policy* is named here (a knob); each side builds the
mask from it with its own code.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int            # seed namespace shared by workloads with the same inputs
    F: int                 # latent frames
    Hh: int                # latent height (tokens)
    W: int                 # latent width (tokens)
    H: int                 # attention heads
    d: int                 # head dimension
    P: int                 # partitions
    steps: int             # denoising steps, including the all-fresh step 0
    sigma: float           # per-step perturbation of the fp32 master tensors
    policy: str            # mask policy for t >= 1: "radius" | "nearest" | "random"
    n_fresh: int           # radius r, or fresh KV partitions per query partition
    pe_amp: float = 2.0    # amplitude of the 3D sinusoidal positional encoding
    dtype: str = "bf16"    # dtype the GPU path consumes
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.F * self.Hh * self.W

    @property
    def S(self) -> int:
        """Rows per partition (the last partition may be shorter)."""
        return -(-self.N // self.P)

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (used for reduced-size test cases)."""
        d = {f: getattr(self, f) for f in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


# The five DiT-shaped workloads.  Seeds depend on cfg_id, so the three mask
# variants of the video workload see identical Q/K/V.
TINY = Workload("tiny", 1, 4, 16, 16, H=2, d=64, P=4, steps=2, sigma=0.05,
                policy="radius", n_fresh=1, dtype="fp32",
                note="1024 tokens; step 1 keeps the diagonal and adjacent partitions fresh")
IMAGE = Workload("image", 2, 1, 128, 128, H=16, d=72, P=8, steps=5, sigma=0.03,
                 policy="nearest", n_fresh=2,
                 note="PixArt-Sigma-shaped 2048px image latent, 75% reuse")
VIDEO_100 = Workload("video_100", 3, 21, 30, 52, H=40, d=128, P=8, steps=5, sigma=0.03,
                     policy="nearest", n_fresh=8, note="Wan-14B-shaped 480p video, all fresh")
VIDEO_50 = Workload("video_50", 3, 21, 30, 52, H=40, d=128, P=8, steps=5, sigma=0.03,
                    policy="nearest", n_fresh=4, note="Wan-14B-shaped 480p video, 50% fresh")
VIDEO_25 = Workload("video_25", 3, 21, 30, 52, H=40, d=128, P=8, steps=5, sigma=0.03,
                    policy="nearest", n_fresh=2, note="Wan-14B-shaped 480p video, 25% fresh")
LONG = Workload("long", 4, 21, 45, 80, H=40, d=128, P=16, steps=4, sigma=0.02,
                policy="nearest", n_fresh=4, note="Wan-14B 720p video, 75600 tokens")
STRESS = Workload("stress", 5, 13, 30, 45, H=48, d=64, P=32, steps=11, sigma=0.03,
                  policy="random", n_fresh=8,
                  note="ragged last partition, seeded random 25% fresh mask per step")

WORKLOADS = {w.name: w for w in (TINY, IMAGE, VIDEO_100, VIDEO_50, VIDEO_25, LONG, STRESS)}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
