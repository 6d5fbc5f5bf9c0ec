"""Host logic of the grouped state cache in the C-ABI library (CPU only, no
GPU work): slot counts, COMPUTE/REUSE decisions and t_c bookkeeping against
the oracle's, argument and state checks.  Device pointers here are fake and
never dereferenced: every call tested returns before any launch."""
import ctypes

import numpy as np
import pytest

import synth
from oracle.groups import group_decisions, n_slots, nearest_groups_mask
from oracle.masks import step_mask as oracle_step_mask

import context_state_reuse_amd as lib
from context_state_reuse_amd import binding

MS = binding.DITANGO_MAX_SLOTS


def _u8(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _tab(vals):
    arr = (ctypes.c_void_p * MS)()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


class _FakeG:
    def __init__(self, H=2, N=100, d=64, P=4, g=2):
        self.shape = lib.make_shape(H, N, d, P)
        self.tc = np.zeros((P, MS), np.int32)
        self.st = binding.ditango_gstates_t()
        n = lib.ditango_group_slots(P, g)
        self.rc = binding.lib.ditango_gstates_init(
            ctypes.byref(self.st), ctypes.byref(self.shape), g,
            _tab([0x100000 * (s + 1) for s in range(n)]), _tab([0x8000000 + 0x100000 * s for s in range(n)]),
            ctypes.c_void_p(self.tc.ctypes.data))
        self.P, self.n = P, n


def test_struct_layout():
    # shape (24 B) and three int32, padded to pointer alignment
    assert binding.ditango_gstates_t.O.offset == 40
    assert binding.ditango_gstates_t.LSE.offset == 40 + 8 * MS
    assert binding.ditango_gstates_t.tc.offset == 40 + 16 * MS
    assert ctypes.sizeof(binding.ditango_gstates_t) == 48 + 16 * MS


@pytest.mark.parametrize("P,g,want", [(32, 1, 0), (31, 1, 32), (32, 2, 17), (16, 4, 5), (5, 2, 4), (8, 100, 2),
                                      (1, 1, 2), (0, 2, 0), (4, 0, 0), (33, 4, 0)])
def test_group_slots(P, g, want):
    assert lib.ditango_group_slots(P, g) == want
    if want:
        assert want == n_slots(P, g)


def test_slot_bytes():
    w = synth.get("long")
    shape = lib.make_shape(w.H, w.N, w.d, w.P)
    ob, lb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    tot = binding.lib.ditango_gstates_slot_bytes(ctypes.byref(shape), ctypes.byref(ob), ctypes.byref(lb))
    assert ob.value == w.H * w.P * w.S * w.d * 4 and lb.value == w.H * w.P * w.S * 4   # fp32 OUT and LSE
    assert tot == ob.value + lb.value
    # g = 4: 5 slots per query partition instead of 16 pair slots
    per_pair, _ = lib.ditango_states_bytes(shape)
    assert 5 * ob.value * 16 == 5 * per_pair


def test_init_and_rejections():
    f = _FakeG()
    assert f.rc == 0 and np.all(f.tc == -1) and f.st.g == f.st.g0 == 2 and f.st.S == 25
    assert f.st.O[f.n - 1] and not f.st.O[f.n]
    for g in (0, -1):
        assert _FakeG(g=g).rc == lib.DITANGO_EINVAL
    assert _FakeG(P=32, N=640, g=1).rc == lib.DITANGO_EINVAL      # 33 slots
    assert _FakeG(P=31, N=620, g=1).rc == 0
    st = binding.ditango_gstates_t()
    shape = lib.make_shape(1, 100, 64, 4)
    tc = np.zeros((4, MS), np.int32)
    odd = _tab([0x100008, 0x200000, 0x300000])
    good = _tab([0x100000, 0x200000, 0x300000])
    init = binding.lib.ditango_gstates_init
    assert init(ctypes.byref(st), ctypes.byref(shape), 2, odd, good, ctypes.c_void_p(tc.ctypes.data)) == -1
    assert init(ctypes.byref(st), ctypes.byref(shape), 2, _tab([0x100000]), good,
                ctypes.c_void_p(tc.ctypes.data)) == -1
    assert init(ctypes.byref(st), ctypes.byref(shape), 2, good, good, None) == -1


def test_partial_merge_compose_refuse_empty_slots_before_launch():
    f = _FakeG(P=4, g=2)
    fake = ctypes.c_void_p(0x30000)
    mask = np.eye(4, dtype=np.uint8)
    rc = binding.lib.ditango_group_attn_partial(fake, fake, fake, _u8(mask), ctypes.byref(f.st), None)
    assert rc == lib.DITANGO_ENOCACHE and "never computed" in binding.lib.ditango_last_error().decode()
    assert binding.lib.ditango_group_merge(ctypes.byref(f.st), fake, fake, None) == lib.DITANGO_ENOCACHE
    assert binding.lib.ditango_group_compose(ctypes.byref(f.st), 2, None) == lib.DITANGO_ENOCACHE
    assert binding.lib.ditango_group_compose(ctypes.byref(f.st), 1, None) == lib.DITANGO_EINVAL
    bad = mask.copy()
    bad[0, 1] = 3
    assert binding.lib.ditango_group_attn_partial(fake, fake, fake, _u8(bad), ctypes.byref(f.st),
                                                  None) == lib.DITANGO_EINVAL


@pytest.mark.parametrize("name,g", [("stress", 4), ("stress", 2), ("long", 4), ("video_25", 3), ("image", 8)])
def test_decisions_and_tc_match_oracle(name, g):
    """computed_out and t_c after every step equal the oracle's bookkeeping."""
    w = synth.get(name)
    f = _FakeG(H=1, N=w.N, d=w.d, P=w.P, g=g)
    assert f.rc == 0
    ns = n_slots(w.P, g)
    tc = np.full((w.P, ns), -1)
    rng = np.random.default_rng(3)
    masks = [oracle_step_mask(w, t) for t in range(w.steps)]
    masks += [(rng.random((w.P, w.P)) < p).astype(np.uint8) for p in (0.05, 0.3, 0.7)]
    for t, m in enumerate(masks):
        computed = np.zeros((w.P, ns), np.uint8)
        assert binding.lib.ditango_group_cache_update(ctypes.byref(f.st), _u8(m), t, _u8(computed)) == 0, \
            binding.lib.ditango_last_error()
        dec = group_decisions(m, g)
        assert np.array_equal(computed, dec), (name, t)
        tc[dec == 1] = t
        assert np.array_equal(f.tc[:, :ns], tc) and np.all(f.tc[:, ns:] == -1)


def test_cache_update_checks_and_reset():
    f = _FakeG(P=4, g=2)
    upd = binding.lib.ditango_group_cache_update
    assert upd(ctypes.byref(f.st), _u8(np.eye(4, dtype=np.uint8)), 0, None) == lib.DITANGO_EINVAL
    assert upd(ctypes.byref(f.st), _u8(np.ones((4, 4), np.uint8)), 3, None) == 0
    assert upd(ctypes.byref(f.st), _u8(np.ones((4, 4), np.uint8)), 2, None) == lib.DITANGO_EINVAL
    assert upd(ctypes.byref(f.st), _u8(np.ones((4, 4), np.uint8)), -1, None) == lib.DITANGO_EINVAL
    # reset binds the original slot count again and empties every slot
    f.st.g = 4
    f.st.O[2] = None
    tabs = [_tab([0x100000, 0x200000, 0x300000]), _tab([0x400000, 0x500000, 0x600000])]
    assert binding.lib.ditango_group_reset(ctypes.byref(f.st), tabs[0], tabs[1]) == 0
    assert f.st.g == 2 and f.st.O[2] == 0x300000 and np.all(f.tc == -1)
    assert binding.lib.ditango_group_reset(ctypes.byref(f.st), _tab([0x100000]), tabs[1]) == lib.DITANGO_EINVAL


def test_group_mask_builder_matches_oracle():
    for P in (1, 2, 3, 5, 8, 13, 16, 31, 32):
        for g in (1, 2, 3, 4, 8, 40):
            for n in (0, 1, 2, 3, 40):
                assert np.array_equal(lib.ditango_group_mask_build(P, g, n), nearest_groups_mask(P, g, n)), (P, g, n)


@pytest.mark.parametrize("args", [(0, 2, 1), (33, 2, 1), (8, 0, 1), (8, 2, -1)])
def test_group_mask_builder_rejects(args):
    with pytest.raises(lib.DitangoError) as e:
        lib.ditango_group_mask_build(*args)
    assert e.value.code == lib.DITANGO_EINVAL


def test_memory_trigger_host_checks():
    """ditango_group_fit: nothing to do when the cache fits, EINVAL before
    any work when not even one group fits or k < 2, ENOCACHE when a merge is
    needed over empty slots (all before any launch, so no GPU is used)."""
    f = _FakeG(P=4, g=2)                       # 1 + 2 slots
    sb = binding.lib.ditango_gstates_slot_bytes(ctypes.byref(f.st.shape), None, None)
    n = ctypes.c_int32(-1)
    fit = binding.lib.ditango_group_fit
    assert fit(ctypes.byref(f.st), 3 * sb, 2, None, ctypes.byref(n)) == 0 and n.value == 0 and f.st.g == 2
    assert fit(ctypes.byref(f.st), 2 * sb - 1, 2, None, ctypes.byref(n)) == lib.DITANGO_EINVAL and n.value == 0
    assert "budget" in binding.lib.ditango_last_error().decode()
    assert fit(ctypes.byref(f.st), 3 * sb, 1, None, ctypes.byref(n)) == lib.DITANGO_EINVAL
    assert fit(ctypes.byref(f.st), 2 * sb, 2, None, ctypes.byref(n)) == lib.DITANGO_ENOCACHE and n.value == 0
    assert f.st.g == 2
    assert fit(ctypes.byref(f.st), 3 * sb, 2, None, None) == 0          # merges_out may be NULL
