"""The C-ABI library on the CPU: it loads, exports what include/ditango.h
declares, and its host logic (masks, t_c, argument checks) is right.  No
call here launches GPU work."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle.masks import step_mask as oracle_step_mask
from oracle.masks import nearest_mask, radius_mask, random_mask

import context_state_reuse_amd as lib
from context_state_reuse_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ditango.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ditango_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 8
    assert set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(binding.lib, n), n
        ctypes.CDLL(binding._LIB_PATH)[n]  # raises AttributeError if missing


def test_version_and_struct_layout():
    assert lib.ditango_version() == 6
    assert ctypes.sizeof(binding.ditango_shape_t) == 24
    assert binding.ditango_states_t.O.offset == 32 and ctypes.sizeof(binding.ditango_states_t) == 56


STRUCTS = ("ditango_shape_t", "ditango_states_t", "ditango_gstates_t", "ditango_planner_t")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_ctypes_structs_match_the_c_header(tmp_path):
    """Every ctypes mirror has the C compiler's field offsets and sizes."""
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "ditango.h"', "int main(void) {"]
    want = []
    for name in STRUCTS:
        cls = getattr(binding, name)
        lines.append(f'printf("%zu\\n", sizeof({name}));')
        want.append(ctypes.sizeof(cls))
        for field, _ in cls._fields_:
            lines.append(f'printf("%zu\\n", offsetof({name}, {field}));')
            want.append(getattr(cls, field).offset)
    lines.append("return 0; }")
    src, exe = tmp_path / "layout.c", tmp_path / "layout"
    src.write_text("\n".join(lines))
    b = subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stderr
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, timeout=60).stdout.split()]
    assert got == want


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_states_bytes(name):
    w = synth.get(name)
    ob, lb = lib.ditango_states_bytes(lib.make_shape(w.H, w.N, w.d, w.P))
    assert ob == w.H * w.P * w.P * w.S * w.d * 4       # fp32 OUT (the default)
    assert lb == w.H * w.P * w.P * w.S * 4
    ob16, lb16 = lib.ditango_states_bytes(lib.make_shape(w.H, w.N, w.d, w.P, state_dtype="bf16"))
    assert ob16 * 2 == ob and lb16 == lb
    # a bf16 state's OUT row is d values: half the 2*d bf16 values of the K
    # and V rows of a key (attention-state section: a state is about half the
    # size of the KV it summarises)
    assert ob16 // (w.H * w.P * w.P * w.S) == (2 * w.d * 2) // 2


def test_state_dtype_is_checked():
    """Only DITANGO_STATE_F32 (0) and DITANGO_STATE_BF16 (1) are state formats:
    any other value is refused before sizes, binding or launches."""
    assert (lib.DITANGO_STATE_F32, lib.DITANGO_STATE_BF16) == (0, 1)
    with pytest.raises(ValueError):
        lib.make_shape(2, 64, 64, 4, state_dtype="fp16")
    tc = np.zeros(16, np.int32)
    for bad in (-1, 2, 7):
        sh = lib.make_shape(2, 64, 64, 4)
        sh.state_dtype = bad
        with pytest.raises(lib.DitangoError):
            lib.ditango_states_bytes(sh)
        assert "state_dtype" in binding.lib.ditango_last_error().decode()
        st = binding.ditango_states_t()
        rc = binding.lib.ditango_states_init(ctypes.byref(st), ctypes.byref(sh), ctypes.c_void_p(0x10000),
                                             ctypes.c_void_p(0x20000), ctypes.c_void_p(tc.ctypes.data))
        assert rc == lib.DITANGO_EINVAL
        assert binding.lib.ditango_gstates_slot_bytes(ctypes.byref(sh), None, None) == 0
    # a grouped slot's OUT halves with bf16 states, its LSE does not
    o32, l32, o16, l16 = (ctypes.c_size_t() for _ in range(4))
    binding.lib.ditango_gstates_slot_bytes(ctypes.byref(lib.make_shape(2, 64, 72, 4)), ctypes.byref(o32), ctypes.byref(l32))
    binding.lib.ditango_gstates_slot_bytes(ctypes.byref(lib.make_shape(2, 64, 72, 4, state_dtype="bf16")),
                                           ctypes.byref(o16), ctypes.byref(l16))
    assert o32.value == 2 * 4 * 16 * 72 * 4 and o16.value * 2 == o32.value and l16.value == l32.value == 2 * 4 * 16 * 4


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_mask_builder_matches_oracle(name):
    w = synth.get(name)
    for t in range(w.steps):
        assert np.array_equal(lib.workload_mask(w, t), oracle_step_mask(w, t)), (name, t)


def test_mask_builder_policies_sweep():
    for P in (1, 2, 3, 5, 8, 16, 31, 32):
        for n in range(0, P + 1):
            assert np.array_equal(lib.ditango_mask_build("radius", P, n), radius_mask(P, n))
        for n in range(1, P + 1):
            assert np.array_equal(lib.ditango_mask_build("nearest", P, n), nearest_mask(P, n))
            for seed in (0, 1, 12345, 2**63 + 7):
                assert np.array_equal(lib.ditango_mask_build("random", P, n, seed, 1), random_mask(P, n, seed + 1))
        assert lib.ditango_mask_build("all", P).sum() == P * P
        assert lib.ditango_mask_build("none", P).sum() == 0


@pytest.mark.parametrize("args", [("nearest", 8, 0), ("nearest", 8, 9), ("random", 8, 0),
                                  ("radius", 8, -1), ("all", 33, 0), ("all", 0, 0), (9, 4, 1)])
def test_mask_builder_rejects(args):
    with pytest.raises(lib.DitangoError) as e:
        lib.ditango_mask_build(*args)
    assert e.value.code == lib.DITANGO_EINVAL


def test_mask_builder_step0_is_anchor_for_every_policy():
    # step 0 is all fresh whatever the policy and its count; the seed is
    # seed + step from step 1 on
    for pol, n in (("radius", 0), ("nearest", 9), ("random", 0), ("none", 0), ("all", 0)):
        assert lib.ditango_mask_build(pol, 8, n, 5, 0).sum() == 64
    assert np.array_equal(lib.ditango_mask_build("random", 8, 3, 1000, 4), random_mask(8, 3, 1004))
    with pytest.raises(lib.DitangoError):
        lib.ditango_mask_build("nearest", 8, 2, 0, -1)
    with pytest.raises(lib.DitangoError):
        lib.ditango_mask_build(9, 8, 2, 0, 0)


@pytest.mark.parametrize("H,N,d,P", [(1, 10, 96, 2), (1, 10, 64, 0), (1, 10, 64, 33), (0, 10, 64, 2),
                                     (1, 3, 64, 4), (1, 10, 64, 6), (1, 2**30 // 128, 128, 8),
                                     (1, 2**30 // 64, 64, 8), (1, 2**30 // 72 + 1, 72, 8)])
def test_shape_rejected(H, N, d, P):
    ob = ctypes.c_size_t(0)
    assert binding.lib.ditango_states_bytes(ctypes.byref(lib.make_shape(H, N, d, P)), ctypes.byref(ob), None) == 0
    assert binding.lib.ditango_last_error()


def test_shape_at_the_size_limit_accepted():
    # K/V of one head are addressed with 32-bit byte offsets: N * d < 2^30
    # (N * d = 2^30 exactly is rejected above)
    ob = ctypes.c_size_t(0)
    for N, d in ((2**30 // 128 - 1, 128), (2**30 // 64 - 1, 64), (2**30 // 72, 72)):
        assert N * d < 2**30
        assert binding.lib.ditango_states_bytes(ctypes.byref(lib.make_shape(1, N, d, 8)),
                                                ctypes.byref(ob), None) > 0


class _FakeStates:
    """A states struct bound to fake (never dereferenced) device addresses."""

    def __init__(self, H=2, N=100, d=64, P=4):
        self.shape = lib.make_shape(H, N, d, P)
        self.tc = np.zeros(P * P, np.int32)
        self.st = binding.ditango_states_t()
        rc = binding.lib.ditango_states_init(ctypes.byref(self.st), ctypes.byref(self.shape),
                                             ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000),
                                             ctypes.c_void_p(self.tc.ctypes.data))
        assert rc == 0
        self.P = P


def _u8(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def test_init_marks_all_pairs_empty():
    f = _FakeStates()
    assert np.all(f.tc == -1) and f.st.S == 25


def test_partial_refuses_reuse_of_empty_pair_before_launch():
    f = _FakeStates()
    mask = radius_mask(4, 1)
    fake = ctypes.c_void_p(0x30000)
    rc = binding.lib.ditango_attn_partial(fake, fake, fake, _u8(mask), ctypes.byref(f.st), None)
    assert rc == lib.DITANGO_ENOCACHE
    assert "never computed" in binding.lib.ditango_last_error().decode()


def test_partial_and_merge_argument_checks():
    f = _FakeStates()
    fake = ctypes.c_void_p(0x30000)
    ones = np.ones((4, 4), np.uint8)
    bad = ones.copy()
    bad[1, 2] = 2
    assert binding.lib.ditango_attn_partial(fake, fake, fake, _u8(bad), ctypes.byref(f.st), None) == lib.DITANGO_EINVAL
    assert binding.lib.ditango_attn_partial(None, fake, fake, _u8(ones), ctypes.byref(f.st), None) == lib.DITANGO_EINVAL
    odd = ctypes.c_void_p(0x30002)
    assert binding.lib.ditango_attn_partial(odd, fake, fake, _u8(ones), ctypes.byref(f.st), None) == lib.DITANGO_EINVAL
    # merge before any state exists
    assert binding.lib.ditango_state_merge(ctypes.byref(f.st), fake, fake, None) == lib.DITANGO_ENOCACHE
    f.st.S = 24
    assert binding.lib.ditango_state_merge(ctypes.byref(f.st), fake, fake, None) == lib.DITANGO_EINVAL


def test_cache_update_bookkeeping():
    f = _FakeStates(P=4)
    upd = binding.lib.ditango_state_cache_update
    reused = np.zeros((4, 4), np.uint8)
    m1 = radius_mask(4, 1)
    # reusing a never-computed pair is refused
    assert upd(ctypes.byref(f.st), _u8(m1), 0, _u8(reused)) == lib.DITANGO_EINVAL
    assert np.all(f.tc == -1)
    # anchor
    assert upd(ctypes.byref(f.st), _u8(np.ones((4, 4), np.uint8)), 0, _u8(reused)) == 0
    assert np.all(f.tc == 0) and reused.sum() == 0
    assert upd(ctypes.byref(f.st), _u8(m1), 1, _u8(reused)) == 0
    assert np.array_equal(reused, 1 - m1)
    want = np.where(m1.ravel() == 1, 1, 0)
    assert np.array_equal(f.tc, want)
    m0 = radius_mask(4, 0)
    assert upd(ctypes.byref(f.st), _u8(m0), 2, None) == 0
    want[m0.ravel() == 1] = 2
    assert np.array_equal(f.tc, want)
    # time does not run backwards, steps are non-negative
    assert upd(ctypes.byref(f.st), _u8(m0), 1, None) == lib.DITANGO_EINVAL
    assert upd(ctypes.byref(f.st), _u8(m0), -1, None) == lib.DITANGO_EINVAL
    # an anchor mid-run resets every t_c
    assert upd(ctypes.byref(f.st), _u8(np.ones((4, 4), np.uint8)), 5, None) == 0
    assert np.all(f.tc == 5)


def test_cache_update_matches_oracle_tc_over_a_workload():
    """t_c after every step equals the oracle's bookkeeping (stress workload masks)."""
    from oracle.reuse import StateReuseOracle
    w = synth.get("stress")
    f = _FakeStates(H=1, N=w.N, d=64, P=w.P)
    orc = StateReuseOracle(w.N, w.P, w.d, rows=[0])  # one row: bookkeeping only
    for t in range(w.steps):
        m = oracle_step_mask(w, t)
        assert binding.lib.ditango_state_cache_update(ctypes.byref(f.st), _u8(m), t, None) == 0
        orc.tc[m == 1] = t
        assert np.array_equal(f.tc.reshape(w.P, w.P), orc.tc)


def test_window_residual_merge_checks_before_launch():
    f = _FakeStates(P=4)
    wr = binding.lib.ditango_window_residual_merge
    fake = ctypes.c_void_p(0x30000)
    win = radius_mask(4, 1)
    # FULL needs every pair; nothing is computed yet
    assert wr(ctypes.byref(f.st), _u8(win), lib.DITANGO_WR_FULL, fake, fake, fake, None) == lib.DITANGO_ENOCACHE
    # WINDOW needs only the window pairs: still missing here
    assert wr(ctypes.byref(f.st), _u8(win), lib.DITANGO_WR_WINDOW, fake, fake, fake, None) == lib.DITANGO_ENOCACHE
    empty = win.copy()
    empty[1] = 0
    assert wr(ctypes.byref(f.st), _u8(empty), lib.DITANGO_WR_WINDOW, fake, fake, fake, None) == lib.DITANGO_EINVAL
    assert wr(ctypes.byref(f.st), _u8(win), 7, fake, fake, fake, None) == lib.DITANGO_EINVAL
    assert wr(ctypes.byref(f.st), _u8(win), lib.DITANGO_WR_FULL, None, fake, fake, None) == lib.DITANGO_EINVAL
    odd = ctypes.c_void_p(0x30004)
    assert wr(ctypes.byref(f.st), _u8(win), lib.DITANGO_WR_FULL, odd, fake, fake, None) == lib.DITANGO_EINVAL


def test_step_checks_everything_before_work():
    f = _FakeStates(P=4)
    fake = ctypes.c_void_p(0x30000)
    step = binding.lib.ditango_step
    m1 = radius_mask(4, 1)
    # a REUSE pair was never computed: refused, t_c untouched
    assert step(fake, fake, fake, _u8(m1), 0, ctypes.byref(f.st), fake, fake, None, None) == lib.DITANGO_ENOCACHE
    assert np.all(f.tc == -1)
    f.tc[:] = 3
    assert step(fake, fake, fake, _u8(m1), 2, ctypes.byref(f.st), fake, fake, None, None) == lib.DITANGO_EINVAL
    assert step(fake, fake, fake, _u8(m1), 4, ctypes.byref(f.st), None, fake, None, None) == lib.DITANGO_EINVAL
    assert np.all(f.tc == 3)


def test_sig_drift_argument_checks():
    """Every refusal happens before a launch: P outside 1..32 (the pair list
    holds 32 x 32 entries), H*d beyond 2^31 - 1, NULL tables, a bad select."""
    drift = binding.lib.ditango_sig_drift
    fake = ctypes.c_void_p(0x30000)
    sel33 = np.ones((33, 33), np.uint8)
    assert drift(fake, fake, 2, 33, 64, binding._u8(sel33), fake, None) == lib.DITANGO_EINVAL
    assert "P=33" in binding.lib.ditango_last_error().decode()
    sel = np.ones((4, 4), np.uint8)
    assert drift(fake, fake, 2, 0, 64, binding._u8(sel), fake, None) == lib.DITANGO_EINVAL
    assert drift(fake, fake, 1 << 16, 4, 1 << 15, binding._u8(sel), fake, None) == lib.DITANGO_EINVAL
    assert drift(None, fake, 2, 4, 64, binding._u8(sel), fake, None) == lib.DITANGO_EINVAL
    assert drift(fake, fake, 2, 4, 64, binding._u8(sel), None, None) == lib.DITANGO_EINVAL
    assert drift(fake, fake, 0, 4, 64, binding._u8(sel), fake, None) == lib.DITANGO_EINVAL
    bad = sel.copy()
    bad[2, 3] = 7
    assert drift(fake, fake, 2, 4, 64, binding._u8(bad), fake, None) == lib.DITANGO_EINVAL
    assert drift(fake, fake, 2, 4, 64, None, fake, None) == lib.DITANGO_EINVAL


def test_evicted_pair_is_refused_until_computed_again():
    """A caller that drops a cached state (t_c set back to -1, e.g. to free
    memory) cannot reuse it: the next step that marks it REUSE is refused
    before any launch, and a step that computes it fresh restores it."""
    f = _FakeStates(P=4)
    upd = binding.lib.ditango_state_cache_update
    fake = ctypes.c_void_p(0x30000)
    ones = np.ones((4, 4), np.uint8)
    assert upd(ctypes.byref(f.st), _u8(ones), 0, None) == 0          # anchor
    m1 = radius_mask(4, 1)
    assert upd(ctypes.byref(f.st), _u8(m1), 1, None) == 0
    f.tc[0 * 4 + 3] = -1                                              # evict pair (0, 3), reused by m1
    for call in (lambda: binding.lib.ditango_attn_partial(fake, fake, fake, _u8(m1), ctypes.byref(f.st), None),
                 lambda: binding.lib.ditango_step(fake, fake, fake, _u8(m1), 2, ctypes.byref(f.st), fake, fake,
                                                  None, None),
                 lambda: binding.lib.ditango_state_merge(ctypes.byref(f.st), fake, fake, None)):
        assert call() == lib.DITANGO_ENOCACHE
        assert "(q=0, k=3)" in binding.lib.ditango_last_error().decode()
    tc_before = f.tc.copy()
    assert upd(ctypes.byref(f.st), _u8(m1), 2, None) == lib.DITANGO_EINVAL
    assert np.array_equal(f.tc, tc_before)                            # a refused commit changes nothing
    # computing the pair again makes the cache whole
    m2 = m1.copy()
    m2[0, 3] = 1
    assert upd(ctypes.byref(f.st), _u8(m2), 2, None) == 0
    assert f.tc[3] == 2 and (f.tc >= 0).all()
    assert upd(ctypes.byref(f.st), _u8(m1), 3, None) == 0
