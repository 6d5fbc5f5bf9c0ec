"""fp64 CPU oracle for partitioned attention with selective state reuse.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The library and its
Python binding never call it, and it shares no code with them: it reads the
seeded inputs from ``synth`` and nothing else.

Everything is written from DiTango: Cost-Effective Parallel Diffusion
Generation with Selective Attention State Reuse (the DiTango page):

* ``state``  -- the attention state (OUT, LSE) of a query block against one
  key partition, and its composition (Eq. 4);
* ``masks``  -- per-step COMPUTE/REUSE selection masks for the workloads;
* ``reuse``  -- the selective compute-and-reuse step with its state cache and
  last-computation timestamps t_c.

Every function computes in float64 with plain NumPy (matrix products, exp,
log); nothing is blocked, fused or reordered beyond the definitions.

Parity pins: every function here is pinned by the CPU tests (brute-force
attention, closed forms, the composition laws, the reuse special cases, the
CP=4 rank-0 example of Fig. 6 and the published SplitMix64 outputs).
"""
from .state import compose, compose2, partial_state, partition_bounds  # noqa: F401
from .masks import SplitMix64, step_mask  # noqa: F401
from .reuse import StateReuseOracle, run_workload  # noqa: F401
