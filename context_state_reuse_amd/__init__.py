"""Partitioned softmax attention with selective attention-state reuse on MI355X.

Python face of libditango.so (C ABI in include/ditango.h).  All work runs in
the library's HIP kernels for gfx950; this package only marshals torch
tensors, host masks and streams into the C calls.
"""
from .binding import (DITANGO_EHIP, DITANGO_EINVAL, DITANGO_ENOCACHE,  # noqa: F401
                      DITANGO_MASK_ALL, DITANGO_MASK_NEAREST, DITANGO_MASK_NONE,
                      DITANGO_MASK_RADIUS, DITANGO_MASK_RANDOM, DITANGO_OK, EXPORTED,
                      DITANGO_MAX_SLOTS, DITANGO_STATE_BF16, DITANGO_STATE_F32, DITANGO_WR_FULL, DITANGO_WR_WINDOW, DitangoError, GroupedStateCache, PlannedSteps, Planner, StateCache,
                      ditango_attn_partial, ditango_attn_partial_merge, ditango_group_attn_partial, ditango_group_attn_partial_merge, ditango_pair_stats, ditango_sig_drift, ditango_group_cache_update,
                      ditango_group_compose, ditango_group_mask_build, ditango_group_merge,
                      ditango_group_slots,
                      group_slot_keys, group_slot_live,
                      ditango_mask_build, ditango_state_cache_update, ditango_state_merge,
                      ditango_states_bytes, ditango_step, ditango_version, ditango_window_residual_merge,
                      make_shape,
                      workload_mask)
