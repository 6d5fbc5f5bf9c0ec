"""ctypes binding of libditango.so: argument marshalling only.

The functions keep the C names of include/ditango.h.  Torch tensors supply
device memory and the current HIP stream; every computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built,
importing this module raises.

torch is imported before the library is opened: torch ships its own HIP
runtime under the same soname (libamdhip64.so.7) as the system one the
library was linked against, and loading torch first makes both use torch's
copy, so the process has a single HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  -- must precede the library: one HIP runtime per process

# DITANGO_LIBRARY may name another build of the same sources (a variant
# compiled with different tile parameters, for side-by-side measurement).
_LIB_PATH = os.environ.get("DITANGO_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libditango.so")

DITANGO_OK = 0
DITANGO_EINVAL = -1
DITANGO_ENOCACHE = -2
DITANGO_EHIP = -3
DITANGO_MAX_P = 32
DITANGO_MAX_SLOTS = 32

DITANGO_MASK_ALL = 0
DITANGO_MASK_NONE = 1
DITANGO_MASK_RADIUS = 2
DITANGO_MASK_NEAREST = 3
DITANGO_MASK_RANDOM = 4

MASK_POLICIES = {"all": DITANGO_MASK_ALL, "none": DITANGO_MASK_NONE, "radius": DITANGO_MASK_RADIUS,
                 "nearest": DITANGO_MASK_NEAREST, "random": DITANGO_MASK_RANDOM}

EXPORTED = ("ditango_states_bytes", "ditango_states_init", "ditango_attn_partial",
            "ditango_state_cache_update", "ditango_state_merge", "ditango_mask_build",
            "ditango_last_error", "ditango_version",
            "ditango_group_slots", "ditango_gstates_slot_bytes", "ditango_gstates_init",
            "ditango_group_attn_partial", "ditango_group_attn_partial_merge", "ditango_group_cache_update",
            "ditango_group_merge",
            "ditango_group_compose", "ditango_group_fit", "ditango_group_reset", "ditango_group_mask_build",
            "ditango_window_residual_merge", "ditango_step", "ditango_attn_partial_merge",
            "ditango_pair_stats", "ditango_sig_drift",
            "ditango_planner_init", "ditango_planner_plan", "ditango_planner_update")


class DitangoError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"ditango error {code}: {message}")
        self.code = code


class ditango_shape_t(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("P", ctypes.c_int32), ("scale", ctypes.c_float), ("state_dtype", ctypes.c_int32)]


DITANGO_STATE_F32, DITANGO_STATE_BF16 = 0, 1
STATE_DTYPES = {"fp32": DITANGO_STATE_F32, "bf16": DITANGO_STATE_BF16}


class ditango_states_t(ctypes.Structure):
    _fields_ = [("shape", ditango_shape_t), ("S", ctypes.c_int32), ("O", ctypes.c_void_p),
                ("LSE", ctypes.c_void_p), ("tc", ctypes.c_void_p)]


class ditango_gstates_t(ctypes.Structure):
    _fields_ = [("shape", ditango_shape_t), ("S", ctypes.c_int32), ("g0", ctypes.c_int32), ("g", ctypes.c_int32),
                ("O", ctypes.c_void_p * DITANGO_MAX_SLOTS), ("LSE", ctypes.c_void_p * DITANGO_MAX_SLOTS),
                ("tc", ctypes.c_void_p)]


class ditango_planner_t(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("g", ctypes.c_int32), ("H", ctypes.c_int32), ("warmup", ctypes.c_int32),
                ("target_reuse", ctypes.c_float), ("drift_max", ctypes.c_float),
                ("anchor", ctypes.c_int32), ("n_anchors", ctypes.c_int32), ("last_anchor", ctypes.c_int32),
                ("eps", ctypes.c_double),
                ("D", ctypes.c_double * DITANGO_MAX_P),
                ("W", (ctypes.c_double * DITANGO_MAX_P) * DITANGO_MAX_P),
                ("alpha", (ctypes.c_double * DITANGO_MAX_P) * DITANGO_MAX_P),
                ("Dc", (ctypes.c_double * DITANGO_MAX_P) * DITANGO_MAX_P)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it first (python context_state_reuse_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    missing = [n for n in EXPORTED if not hasattr(lib, n)]
    if missing:
        raise ImportError(f"{_LIB_PATH} lacks {', '.join(missing)}: it predates these sources, rebuild it "
                          f"(python context_state_reuse_amd/build.py)")
    vp, i32, u8p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint8)
    lib.ditango_states_bytes.restype = ctypes.c_size_t
    lib.ditango_states_bytes.argtypes = [ctypes.POINTER(ditango_shape_t), ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.ditango_states_init.restype = ctypes.c_int
    lib.ditango_states_init.argtypes = [ctypes.POINTER(ditango_states_t), ctypes.POINTER(ditango_shape_t),
                                        vp, vp, vp]
    lib.ditango_attn_partial.restype = ctypes.c_int
    lib.ditango_attn_partial.argtypes = [vp, vp, vp, u8p, ctypes.POINTER(ditango_states_t), vp]
    lib.ditango_state_cache_update.restype = ctypes.c_int
    lib.ditango_state_cache_update.argtypes = [ctypes.POINTER(ditango_states_t), u8p, i32, u8p]
    lib.ditango_state_merge.restype = ctypes.c_int
    lib.ditango_state_merge.argtypes = [ctypes.POINTER(ditango_states_t), vp, vp, vp]
    lib.ditango_mask_build.restype = ctypes.c_int
    lib.ditango_mask_build.argtypes = [i32, i32, i32, ctypes.c_uint64, i32, u8p]
    lib.ditango_last_error.restype = ctypes.c_char_p
    lib.ditango_last_error.argtypes = []
    lib.ditango_version.restype = ctypes.c_int32
    lib.ditango_version.argtypes = []
    gst = ctypes.POINTER(ditango_gstates_t)
    ptab = ctypes.POINTER(ctypes.c_void_p)
    lib.ditango_group_slots.restype = ctypes.c_int32
    lib.ditango_group_slots.argtypes = [i32, i32]
    lib.ditango_gstates_slot_bytes.restype = ctypes.c_size_t
    lib.ditango_gstates_slot_bytes.argtypes = [ctypes.POINTER(ditango_shape_t), ctypes.POINTER(ctypes.c_size_t),
                                               ctypes.POINTER(ctypes.c_size_t)]
    lib.ditango_gstates_init.restype = ctypes.c_int
    lib.ditango_gstates_init.argtypes = [gst, ctypes.POINTER(ditango_shape_t), i32, ptab, ptab, vp]
    lib.ditango_group_attn_partial.restype = ctypes.c_int
    lib.ditango_group_attn_partial.argtypes = [vp, vp, vp, u8p, gst, vp]
    lib.ditango_group_attn_partial_merge.restype = ctypes.c_int
    lib.ditango_group_attn_partial_merge.argtypes = [vp, vp, vp, u8p, gst, vp, vp, vp]
    lib.ditango_group_cache_update.restype = ctypes.c_int
    lib.ditango_group_cache_update.argtypes = [gst, u8p, i32, u8p]
    lib.ditango_group_merge.restype = ctypes.c_int
    lib.ditango_group_merge.argtypes = [gst, vp, vp, vp]
    lib.ditango_group_compose.restype = ctypes.c_int
    lib.ditango_group_compose.argtypes = [gst, i32, vp]
    lib.ditango_group_fit.restype = ctypes.c_int
    lib.ditango_group_fit.argtypes = [gst, ctypes.c_size_t, i32, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.ditango_group_reset.restype = ctypes.c_int
    lib.ditango_group_reset.argtypes = [gst, ptab, ptab]
    lib.ditango_group_mask_build.restype = ctypes.c_int
    lib.ditango_group_mask_build.argtypes = [i32, i32, i32, u8p]
    lib.ditango_step.restype = ctypes.c_int
    lib.ditango_step.argtypes = [vp, vp, vp, u8p, i32, ctypes.POINTER(ditango_states_t), vp, vp, u8p, vp]
    lib.ditango_attn_partial_merge.restype = ctypes.c_int
    lib.ditango_attn_partial_merge.argtypes = [vp, vp, vp, u8p, ctypes.POINTER(ditango_states_t), vp, vp, vp]
    lib.ditango_pair_stats.restype = ctypes.c_int
    lib.ditango_pair_stats.argtypes = [ctypes.POINTER(ditango_states_t), vp, u8p, vp, vp, vp]
    plp, f32p = ctypes.POINTER(ditango_planner_t), ctypes.POINTER(ctypes.c_float)
    lib.ditango_sig_drift.restype = ctypes.c_int
    lib.ditango_sig_drift.argtypes = [vp, vp, i32, i32, i32, u8p, vp, vp]
    lib.ditango_planner_init.restype = ctypes.c_int
    lib.ditango_planner_init.argtypes = [plp, i32, i32, i32, ctypes.c_float, ctypes.c_float, i32]
    lib.ditango_planner_plan.restype = ctypes.c_int
    lib.ditango_planner_plan.argtypes = [plp, i32, f32p, u8p, ctypes.POINTER(ctypes.c_int32)]
    lib.ditango_planner_update.restype = ctypes.c_int
    lib.ditango_planner_update.argtypes = [plp, i32, u8p, f32p, f32p]
    lib.ditango_window_residual_merge.restype = ctypes.c_int
    lib.ditango_window_residual_merge.argtypes = [ctypes.POINTER(ditango_states_t), u8p, i32, vp, vp, vp, vp]
    return lib


lib = _load()


def _check(rc: int) -> None:
    if rc != DITANGO_OK:
        raise DitangoError(rc, lib.ditango_last_error().decode())


def _u8(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _mask(mask, P: int) -> np.ndarray:
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
    if m.shape != (P, P):
        raise ValueError(f"mask must be ({P}, {P}), got {m.shape}")
    return m


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _torch_stream(stream):
    """The torch stream for `stream` (None: torch's current one), so that the
    binding's own torch work (fills, copies) is ordered with the launches."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def make_shape(H: int, N: int, d: int, P: int, scale: float | None = None, state_dtype: str = "fp32") -> ditango_shape_t:
    """Layer shape; state_dtype "fp32" (default) or "bf16" is the number
    format of the cached states' OUT."""
    if state_dtype not in STATE_DTYPES:
        raise ValueError(f"state_dtype must be one of {sorted(STATE_DTYPES)}")
    return ditango_shape_t(H, N, d, P, float(1.0 / np.sqrt(d) if scale is None else scale), STATE_DTYPES[state_dtype])


def _torch_state_dtype(shape: ditango_shape_t):
    import torch
    return torch.bfloat16 if shape.state_dtype == DITANGO_STATE_BF16 else torch.float32


def ditango_states_bytes(shape: ditango_shape_t) -> tuple[int, int]:
    ob, lb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    if lib.ditango_states_bytes(ctypes.byref(shape), ctypes.byref(ob), ctypes.byref(lb)) == 0:
        raise DitangoError(DITANGO_EINVAL, lib.ditango_last_error().decode())
    return ob.value, lb.value


class StateCache:
    """The attention-state cache: device O (float32, or bfloat16 with
    state_dtype="bf16") / LSE (float32) slots (torch) and host t_c."""

    def __init__(self, H: int, N: int, d: int, P: int, scale: float | None = None, device="cuda",
                 state_dtype: str = "fp32"):
        import torch
        self.shape = make_shape(H, N, d, P, scale, state_dtype)
        ob, lb = ditango_states_bytes(self.shape)
        S = -(-N // P)
        dt = _torch_state_dtype(self.shape)
        assert ob == H * P * P * S * d * torch.tensor([], dtype=dt).element_size() and lb == H * P * P * S * 4
        self.O = torch.empty((H, P * P, S, d), dtype=dt, device=device)
        self.LSE = torch.empty((H, P * P, S), dtype=torch.float32, device=device)
        self.tc = np.full(P * P, -1, dtype=np.int32)
        self.st = ditango_states_t()
        _check(lib.ditango_states_init(ctypes.byref(self.st), ctypes.byref(self.shape),
                                       ctypes.c_void_p(self.O.data_ptr()), ctypes.c_void_p(self.LSE.data_ptr()),
                                       ctypes.c_void_p(self.tc.ctypes.data)))
        self.H, self.N, self.d, self.P, self.S = H, N, d, P, S

    @property
    def tc_matrix(self) -> np.ndarray:
        return self.tc.reshape(self.P, self.P).copy()


def _qkv(x, cache: StateCache, name: str):
    import torch
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    if tuple(x.shape) != (cache.H, cache.N, cache.d):
        raise ValueError(f"{name} must have shape {(cache.H, cache.N, cache.d)}, got {tuple(x.shape)}")
    return ctypes.c_void_p(x.data_ptr())


def ditango_attn_partial(Q, K, V, mask, cache: StateCache, stream=None) -> None:
    m = _mask(mask, cache.P)
    _check(lib.ditango_attn_partial(_qkv(Q, cache, "Q"), _qkv(K, cache, "K"), _qkv(V, cache, "V"),
                                    _u8(m), ctypes.byref(cache.st), _stream(stream)))


def ditango_state_cache_update(cache: StateCache, mask, step: int) -> np.ndarray:
    m = _mask(mask, cache.P)
    reused = np.zeros((cache.P, cache.P), dtype=np.uint8)
    _check(lib.ditango_state_cache_update(ctypes.byref(cache.st), _u8(m), int(step), _u8(reused)))
    return reused


def ditango_state_merge(cache: StateCache, O=None, LSE=None, stream=None):
    import torch
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=cache.O.device)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=cache.O.device)
    for t, shp, nm in ((O, (cache.H, cache.N, cache.d), "O"), (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_state_merge(ctypes.byref(cache.st), ctypes.c_void_p(O.data_ptr()),
                                   ctypes.c_void_p(LSE.data_ptr()), _stream(stream)))
    return O, LSE


def ditango_step(Q, K, V, mask, step: int, cache: StateCache, O=None, LSE=None, stream=None):
    """One denoising step through the library's own driver: partial attention,
    t_c update and composition.  Returns (O, LSE, reused)."""
    import torch
    m = _mask(mask, cache.P)
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=cache.O.device)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=cache.O.device)
    for t, shp, nm in ((O, (cache.H, cache.N, cache.d), "O"), (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    reused = np.zeros((cache.P, cache.P), dtype=np.uint8)
    _check(lib.ditango_step(_qkv(Q, cache, "Q"), _qkv(K, cache, "K"), _qkv(V, cache, "V"), _u8(m), int(step),
                            ctypes.byref(cache.st), ctypes.c_void_p(O.data_ptr()), ctypes.c_void_p(LSE.data_ptr()),
                            _u8(reused), _stream(stream)))
    return O, LSE, reused


def ditango_attn_partial_merge(Q, K, V, mask, cache: StateCache, O=None, LSE=None, stream=None):
    """Fresh partial attention of the COMPUTE pairs and the composition of
    every row in one launch (t_c unchanged).  Returns (O, LSE)."""
    import torch
    m = _mask(mask, cache.P)
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=cache.O.device)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=cache.O.device)
    for t, shp, nm in ((O, (cache.H, cache.N, cache.d), "O"), (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_attn_partial_merge(_qkv(Q, cache, "Q"), _qkv(K, cache, "K"), _qkv(V, cache, "V"), _u8(m),
                                          ctypes.byref(cache.st), ctypes.c_void_p(O.data_ptr()),
                                          ctypes.c_void_p(LSE.data_ptr()), _stream(stream)))
    return O, LSE


def ditango_pair_stats(cache: StateCache, LSE, select, W=None, SIG=None, stream=None, want_w=True):
    """Per-pair importance W [H][P][P] (every pair; skipped with want_w=False,
    LSE then unused and may be None) and signatures SIG [H][P][P][d] (pairs
    with select = 1; other entries untouched) of the cache, given the merged
    LSE [H][N] of the same contents."""
    import torch
    m = _mask(select, cache.P)
    dev = cache.O.device
    if want_w and W is None:
        W = torch.empty((cache.H, cache.P, cache.P), dtype=torch.float32, device=dev)
    if SIG is None:
        with torch.cuda.stream(_torch_stream(stream)):   # the fill precedes the kernel on its stream
            SIG = torch.zeros((cache.H, cache.P, cache.P, cache.d), dtype=torch.float32, device=dev)
    checks = [(SIG, (cache.H, cache.P, cache.P, cache.d), "SIG")]
    if want_w:
        checks += [(LSE, (cache.H, cache.N), "LSE"), (W, (cache.H, cache.P, cache.P), "W")]
    for t, shp, nm in checks:
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_pair_stats(ctypes.byref(cache.st), ctypes.c_void_p(LSE.data_ptr() if want_w else None),
                                  _u8(m), ctypes.c_void_p(W.data_ptr() if want_w else None),
                                  ctypes.c_void_p(SIG.data_ptr()), _stream(stream)))
    return (W if want_w else None), SIG


def ditango_sig_drift(A, B, select, out=None, stream=None):
    """out[q][k] = ||A - B|| / ||B|| over heads and dims for the selected
    pairs of two signature tables [H][P][P][d] (device float32)."""
    import torch
    H, P, _, d = A.shape
    m = _mask(select, P)
    if out is None:
        with torch.cuda.stream(_torch_stream(stream)):   # the fill precedes the kernel on its stream
            out = torch.zeros((P, P), dtype=torch.float32, device=A.device)
    for t, shp, nm in ((A, (H, P, P, d), "A"), (B, (H, P, P, d), "B"), (out, (P, P), "out")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_sig_drift(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()), int(H), int(P), int(d),
                                 _u8(m), ctypes.c_void_p(out.data_ptr()), _stream(stream)))
    return out


def _f32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


class Planner:
    """Anchor-guided selection (host, ditango_planner_*): decisions from
    per-partition local drifts D [P], head-wise importance W [H][P][P] and
    per-pair drifts e [P][P] (host float32 arrays, the latter two read at
    anchor steps only)."""

    def __init__(self, P: int, g: int, H: int, target_reuse: float, drift_max: float, warmup: int = 2):
        self.P, self.H = P, H
        self.pl = ditango_planner_t()
        _check(lib.ditango_planner_init(ctypes.byref(self.pl), int(P), int(g), int(H), float(target_reuse),
                                        float(drift_max), int(warmup)))

    def plan(self, step: int, drift=None) -> tuple[np.ndarray, bool]:
        D = None if drift is None else np.ascontiguousarray(drift, dtype=np.float32).reshape(self.P)
        mask = np.zeros((self.P, self.P), dtype=np.uint8)
        anchor = ctypes.c_int32(0)
        _check(lib.ditango_planner_plan(ctypes.byref(self.pl), int(step), None if D is None else _f32(D), _u8(mask),
                                        ctypes.byref(anchor)))
        return mask, bool(anchor.value)

    def update(self, step: int, mask, W=None, e=None) -> None:
        m = _mask(mask, self.P)
        if W is not None:
            W = np.ascontiguousarray(W, dtype=np.float32)
            if W.shape != (self.H, self.P, self.P):
                raise ValueError(f"W must have shape {(self.H, self.P, self.P)}")
        if e is not None:
            e = np.ascontiguousarray(e, dtype=np.float32).reshape(self.P, self.P)
        _check(lib.ditango_planner_update(ctypes.byref(self.pl), int(step), _u8(m),
                                          None if W is None else _f32(W), None if e is None else _f32(e)))

    @property
    def eps(self) -> float:
        return float(self.pl.eps)

    @property
    def n_anchors(self) -> int:
        return int(self.pl.n_anchors)

    @property
    def anchor(self) -> bool:
        return bool(self.pl.anchor)


class PlannedSteps:
    """Denoising steps with the planner choosing each step's mask, on one
    stream: the local pairs are computed first and their signatures' drift
    since the last anchor measured; the planner picks the mask; t_c is
    updated, then the other chosen pairs are computed and every row composed
    in one fused launch; the
    signatures of the fresh pairs are refreshed, and at anchor steps the
    importance and every pair's drift against the cache before the step go
    to the planner.  Signature tables stay on the device; only P or P*P
    scalars per step (H*P*P at anchors) reach the host."""

    def __init__(self, cache: StateCache, planner: Planner):
        import torch
        self.cache, self.planner = cache, planner
        dev = cache.O.device
        H, P, d = cache.H, cache.P, cache.d
        self.W = torch.empty((H, P, P), dtype=torch.float32, device=dev)
        self.SIG = torch.zeros((H, P, P, d), dtype=torch.float32, device=dev)      # signatures of the cache
        self.OLD = torch.zeros_like(self.SIG)     # the cache before an anchor step
        self.REF = torch.zeros_like(self.SIG)     # signatures at the last anchor (diagonal used)
        self.DR = torch.zeros((P, P), dtype=torch.float32, device=dev)
        self.O = torch.empty((H, cache.N, d), dtype=torch.float32, device=dev)
        self.LSE = torch.zeros((H, cache.N), dtype=torch.float32, device=dev)
        # the fills above are done before any step uses the tables, on any stream
        torch.cuda.current_stream().synchronize()
        self.eye = np.eye(P, dtype=np.uint8)
        self.off = (1 - self.eye).astype(np.uint8)

    def step(self, t: int, Q, K, V, stream=None):
        """Returns (mask, anchor, O, LSE); O and LSE are this object's buffers.
        Everything runs on `stream` (default: torch's current stream): the
        launches and the table copies alike."""
        import torch
        with torch.cuda.stream(_torch_stream(stream)):
            return self._step(t, Q, K, V, stream)

    def _step(self, t: int, Q, K, V, stream):
        c, pl = self.cache, self.planner
        drift = None
        if pl.n_anchors:
            ditango_attn_partial(Q, K, V, self.eye, c, stream)
            ditango_pair_stats(c, None, self.eye, None, self.SIG, stream, want_w=False)
            ditango_sig_drift(self.SIG, self.REF, self.eye, self.DR, stream)
            drift = self.DR.cpu().numpy().diagonal().copy()   # P*P floats: no gather kernel
        mask, anchor = pl.plan(t, drift)
        if anchor and pl.n_anchors:
            self.OLD.copy_(self.SIG)
        rest = mask.copy()
        if pl.n_anchors:
            rest[self.eye == 1] = 0
        # t_c first (host only), so the local pairs computed above count as
        # cached; then the other chosen pairs and the composition of every row
        # in one fused launch
        ditango_state_cache_update(c, mask, t)
        ditango_attn_partial_merge(Q, K, V, rest, c, self.O, self.LSE, stream)
        # signatures of the pairs computed after the plan (the local ones, when
        # already refreshed above, are not read again); the importance of every
        # pair at an anchor
        refresh = rest if pl.n_anchors else mask
        if anchor or rest.any():
            ditango_pair_stats(c, self.LSE, refresh, self.W, self.SIG, stream, want_w=anchor)
        if anchor:
            e = None
            if pl.n_anchors:
                ditango_sig_drift(self.SIG, self.OLD, self.off, self.DR, stream)
                e = self.DR.cpu().numpy()
            self.REF.copy_(self.SIG)
            pl.update(t, mask, self.W.cpu().numpy(), e)
        else:
            pl.update(t, mask)
        return mask, anchor, self.O, self.LSE


DITANGO_WR_FULL = 0
DITANGO_WR_WINDOW = 1


def ditango_window_residual_merge(cache: StateCache, window, mode: int, R, O=None, LSE=None, stream=None):
    """Window attention with residual sharing: FULL writes O, LSE and R; WINDOW reads R."""
    import torch
    w = _mask(window, cache.P)
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=cache.O.device)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=cache.O.device)
    for t, shp, nm in ((R, (cache.H, cache.N, cache.d), "R"), (O, (cache.H, cache.N, cache.d), "O"),
                       (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_window_residual_merge(ctypes.byref(cache.st), _u8(w), int(mode), ctypes.c_void_p(R.data_ptr()),
                                             ctypes.c_void_p(O.data_ptr()), ctypes.c_void_p(LSE.data_ptr()),
                                             _stream(stream)))
    return O, LSE


def ditango_mask_build(policy, P: int, n: int = 0, seed: int = 0, step: int = 1) -> np.ndarray:
    """Mask of step `step` (0: the all-fresh anchor) under `policy`; the
    random policy draws with seed + step."""
    pol = MASK_POLICIES[policy] if isinstance(policy, str) else int(policy)
    out = np.zeros((P, P), dtype=np.uint8) if 1 <= P <= DITANGO_MAX_P else np.zeros(1, dtype=np.uint8)
    _check(lib.ditango_mask_build(pol, int(P), int(n), ctypes.c_uint64(seed & ((1 << 64) - 1)), int(step), _u8(out)))
    return out


def ditango_version() -> int:
    return int(lib.ditango_version())


def workload_mask(w, t: int) -> np.ndarray:
    """Mask of step t of a workload, built by the library (step 0: all fresh)."""
    return ditango_mask_build(w.policy, w.P, w.n_fresh, 1000 * w.cfg_id, t)


# ------------------------------------------------------------ grouped cache

def ditango_group_slots(P: int, g: int) -> int:
    return int(lib.ditango_group_slots(int(P), int(g)))


def group_slot_range(P: int, g: int, q: int, s: int) -> tuple[int, int]:
    """Partitions [a, b) spanned by slot s of query partition q (slot 0: q itself)."""
    if s == 0:
        return q, q + 1
    a = (s - 1) * g
    return a, min(a + g, P)


def group_slot_live(P: int, g: int, q: int, s: int) -> bool:
    """The slot holds a state (a group that is {q} alone does not)."""
    a, b = group_slot_range(P, g, q, s)
    return s == 0 or b - a > 1 or a != q


def group_slot_keys(N: int, P: int, g: int, q: int, s: int) -> int:
    """Keys whose attention the state of slot s of q covers."""
    S = -(-N // P)
    a, b = group_slot_range(P, g, q, s)
    n = min(b * S, N) - a * S
    if s != 0 and a <= q < b:
        n -= min(S, N - q * S)
    return n


def _ptab(ptrs):
    arr = (ctypes.c_void_p * DITANGO_MAX_SLOTS)()
    for i, x in enumerate(ptrs):
        arr[i] = x
    return arr


class GroupedStateCache:
    """Grouped, composed state cache: one device tensor pair per slot.

    Slot s of query partition q (0 = the local pair, 1 + j = group j of g
    adjacent partitions without q) holds rows [h][q][S][d].  A group merge
    (``compose``) releases the slots it no longer needs, so their memory
    returns to the allocator; ``reset`` re-creates them for an anchor step.
    """

    def __init__(self, H: int, N: int, d: int, P: int, g: int, scale: float | None = None, device="cuda",
                 state_dtype: str = "fp32"):
        self.shape = make_shape(H, N, d, P, scale, state_dtype)
        self.H, self.N, self.d, self.P = H, N, d, P
        self.S = -(-N // P)
        self.device = device
        n = ditango_group_slots(P, g)
        if n == 0:
            raise DitangoError(DITANGO_EINVAL, f"group size {g} is invalid for P={P}")
        self.O = [self._slot_o() for _ in range(n)]
        self.LSE = [self._slot_l() for _ in range(n)]
        self.tc = np.full((P, DITANGO_MAX_SLOTS), -1, dtype=np.int32)
        self.st = ditango_gstates_t()
        _check(lib.ditango_gstates_init(ctypes.byref(self.st), ctypes.byref(self.shape), int(g),
                                        _ptab([t.data_ptr() for t in self.O]),
                                        _ptab([t.data_ptr() for t in self.LSE]),
                                        ctypes.c_void_p(self.tc.ctypes.data)))

    def _slot_o(self):
        import torch
        return torch.empty((self.H, self.P, self.S, self.d), dtype=_torch_state_dtype(self.shape), device=self.device)

    def _slot_l(self):
        import torch
        return torch.empty((self.H, self.P, self.S), dtype=torch.float32, device=self.device)

    @property
    def g(self) -> int:
        return int(self.st.g)

    @property
    def n_slots(self) -> int:
        return ditango_group_slots(self.P, self.g)

    @property
    def tc_matrix(self) -> np.ndarray:
        return self.tc[:, :self.n_slots].copy()

    @property
    def device_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.O + self.LSE)

    def compose(self, k: int = 2, stream=None, after=None) -> None:
        """Dynamic Group State Compose: group size g -> k g; frees released slots.

        ``after`` (optional) is called right after the work is enqueued,
        before the buffers are released (e.g. to record a timing event)."""
        import torch
        _check(lib.ditango_group_compose(ctypes.byref(self.st), int(k), _stream(stream)))
        if after is not None:
            after()
        n = self.n_slots
        if len(self.O) > n:
            # the released buffers are read by the queued group merges
            torch.cuda.synchronize()
            del self.O[n:], self.LSE[n:]

    def fit(self, budget_bytes: int, k: int = 2, stream=None) -> int:
        """Memory trigger of Dynamic Group State Compose: merge groups k at a
        time while the cache's slot memory exceeds budget_bytes; frees the
        released slots.  Returns the number of merges."""
        import torch
        merges = ctypes.c_int32(0)
        _check(lib.ditango_group_fit(ctypes.byref(self.st), ctypes.c_size_t(int(budget_bytes)), int(k),
                                     _stream(stream), ctypes.byref(merges)))
        n = self.n_slots
        if len(self.O) > n:
            torch.cuda.synchronize()
            del self.O[n:], self.LSE[n:]
        return int(merges.value)

    def reset(self) -> None:
        """Back to the original group size with every slot empty (before an anchor step)."""
        n = ditango_group_slots(self.P, int(self.st.g0))
        while len(self.O) < n:
            self.O.append(self._slot_o())
            self.LSE.append(self._slot_l())
        _check(lib.ditango_group_reset(ctypes.byref(self.st), _ptab([t.data_ptr() for t in self.O]),
                                       _ptab([t.data_ptr() for t in self.LSE])))


def ditango_group_attn_partial(Q, K, V, mask, cache: GroupedStateCache, stream=None) -> None:
    m = _mask(mask, cache.P)
    _check(lib.ditango_group_attn_partial(_qkv(Q, cache, "Q"), _qkv(K, cache, "K"), _qkv(V, cache, "V"),
                                          _u8(m), ctypes.byref(cache.st), _stream(stream)))


def ditango_group_cache_update(cache: GroupedStateCache, mask, step: int) -> np.ndarray:
    m = _mask(mask, cache.P)
    computed = np.zeros((cache.P, cache.n_slots), dtype=np.uint8)
    _check(lib.ditango_group_cache_update(ctypes.byref(cache.st), _u8(m), int(step), _u8(computed)))
    return computed


def _group_out(cache, O, LSE):
    import torch
    dev = cache.O[0].device
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=dev)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=dev)
    for t, shp, nm in ((O, (cache.H, cache.N, cache.d), "O"), (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    return O, LSE


def ditango_group_attn_partial_merge(Q, K, V, mask, cache: GroupedStateCache, O=None, LSE=None, stream=None):
    """Fresh states of the COMPUTE slots and the composition of every row in
    one launch (t_c unchanged).  Returns (O, LSE)."""
    m = _mask(mask, cache.P)
    O, LSE = _group_out(cache, O, LSE)
    _check(lib.ditango_group_attn_partial_merge(_qkv(Q, cache, "Q"), _qkv(K, cache, "K"), _qkv(V, cache, "V"), _u8(m),
                                                ctypes.byref(cache.st), ctypes.c_void_p(O.data_ptr()),
                                                ctypes.c_void_p(LSE.data_ptr()), _stream(stream)))
    return O, LSE


def ditango_group_merge(cache: GroupedStateCache, O=None, LSE=None, stream=None):
    import torch
    dev = cache.O[0].device
    if O is None:
        O = torch.empty((cache.H, cache.N, cache.d), dtype=torch.float32, device=dev)
    if LSE is None:
        LSE = torch.empty((cache.H, cache.N), dtype=torch.float32, device=dev)
    for t, shp, nm in ((O, (cache.H, cache.N, cache.d), "O"), (LSE, (cache.H, cache.N), "LSE")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == shp):
            raise ValueError(f"{nm} must be a contiguous float32 device tensor of shape {shp}")
    _check(lib.ditango_group_merge(ctypes.byref(cache.st), ctypes.c_void_p(O.data_ptr()),
                                   ctypes.c_void_p(LSE.data_ptr()), _stream(stream)))
    return O, LSE


def ditango_group_compose(cache: GroupedStateCache, k: int = 2, stream=None) -> None:
    cache.compose(k, stream)


def ditango_group_mask_build(P: int, g: int, n: int) -> np.ndarray:
    """Pair mask selecting, per query partition, the local pair and the n nearest groups."""
    out = np.zeros((P, P), dtype=np.uint8) if 1 <= P <= DITANGO_MAX_P else np.zeros(1, dtype=np.uint8)
    _check(lib.ditango_group_mask_build(int(P), int(g), int(n), _u8(out)))
    return out
