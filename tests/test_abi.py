"""C ABI checks that need no GPU: the library loads, exports every entry point the header
declares, computes layouts, and rejects bad arguments on the host before any HIP call.

States with batch = 0 are fully valid and every call on them is a no-op, so the state-machine
errors (pending drafts, capacity, rollback without drafts) can be driven without a device; fake
device addresses are never dereferenced because validation fails (or there is no work) first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_replay.h")

bd = pytest.importorskip("ssm_decode_state_amd.binding",
                         reason="libssm_replay.so not built (run __graft_entry__.build())")

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(bd._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.EXPORTS)


def test_abi_version_and_status_strings():
    assert bd.ssm_abi_version() == 5
    for s in range(-7, 1):
        assert bd.ssm_status_string(s) not in ("", "unknown status")
    assert bd.ssm_status_string(-99) == "unknown status"


def cfg(**kw):
    base = dict(kind=bd.SSM_MAMBA2, batch=256, heads=128, groups=128, dim_p=64, dim_n=128,
                window=16, max_draft=1, in_dtype=bd.SSM_IN_BF16, readcopy=bd.SSM_RC_NONE)
    base.update(kw)
    return bd.make_config(**base)


def test_layout_serving_shape():
    lay = bd.ssm_layout_query(cfg())
    assert lay.ring_cap == 16
    assert lay.off_ckpt == 0
    ck = 256 * 128 * 64 * 128 * 4
    assert lay.off_ring[0] >= ck
    offs = [lay.off_ckpt, lay.off_rc_codes, lay.off_ring[0], lay.off_ring[1], lay.off_ring[2],
            lay.off_ring[3], lay.off_ptr]
    assert all(o % 256 == 0 for o in offs)
    assert offs == sorted(offs)
    # the ring keeps x, B and dt; C enters only its own token's output and has no ring
    assert lay.off_ring[1] - lay.off_ring[0] == 256 * 128 * 16 * 64 * 2
    assert lay.off_ring[2] - lay.off_ring[1] == 256 * 128 * 16 * 128 * 2
    assert lay.off_ring[3] == lay.off_ring[2]
    assert lay.off_ptr - lay.off_ring[3] == 256 * 128 * 16 * 4
    assert lay.off_flags >= lay.off_ptr + 256 * 128 * 16 and lay.off_flags % 256 == 0
    assert lay.ckpt_slots == 256 and lay.off_refcnt >= lay.off_flags + 4
    assert lay.total_bytes >= lay.off_refcnt + 256 * 4
    spec = bd.ssm_layout_query(cfg(max_draft=4))
    assert spec.ring_cap == 19


def test_layout_shared_checkpoints():
    # sharing doubles the checkpoint slots (tiles and read copy); rings and pointers are unchanged
    plain = bd.ssm_layout_query(cfg(readcopy=bd.SSM_RC_FP8_ROW))
    shared = bd.ssm_layout_query(cfg(readcopy=bd.SSM_RC_FP8_ROW, share_ckpt=1))
    assert shared.ckpt_slots == 512
    assert shared.off_rc_codes == 2 * 256 * 128 * 64 * 128 * 4
    assert shared.off_rc_scale - shared.off_rc_codes == 2 * 256 * 128 * 64 * 128
    assert shared.off_ptr - shared.off_ring[0] == plain.off_ptr - plain.off_ring[0]
    assert shared.total_bytes >= shared.off_refcnt + 512 * 4


def test_layout_gdn_read_copies():
    c = cfg(kind=bd.SSM_GDN, heads=32, groups=32, dim_p=128, dim_n=128)
    f8 = bd.ssm_layout_query(bd.make_config(**{**{f: getattr(c, f) for f, _ in c._fields_},
                                              "readcopy": bd.SSM_RC_FP8_ROW}))
    assert f8.off_rc_scale - f8.off_rc_codes == 256 * 32 * 128 * 128
    f4 = bd.ssm_layout_query(bd.make_config(**{**{f: getattr(c, f) for f, _ in c._fields_},
                                              "readcopy": bd.SSM_RC_FP4_B16}))
    assert f4.off_rc_tscale - f4.off_rc_scale == 256 * 32 * 128 * 8


def test_layout_kda_gate_ring():
    c = dict(kind=bd.SSM_KDA, heads=32, groups=32, dim_p=128, dim_n=128)
    kda = bd.ssm_layout_query(cfg(**c))
    gdn = bd.ssm_layout_query(cfg(**{**c, "kind": bd.SSM_GDN}))
    # KDA keeps dk log-decays per entry: the g ring is dk times the GDN one
    assert kda.off_ptr - kda.off_ring[4] == 256 * 32 * 16 * 128 * 4
    assert gdn.off_ptr - gdn.off_ring[4] == 256 * 32 * 16 * 4
    # k, v, beta and g are buffered; q enters only its own token's output and has no ring
    for lay in (kda, gdn):
        assert lay.off_ring[0] == lay.off_ring[1]
        assert lay.off_ring[2] - lay.off_ring[1] == 256 * 32 * 16 * 128 * 2


def test_layout_read_copies():
    f8 = bd.ssm_layout_query(cfg(readcopy=bd.SSM_RC_FP8_ROW))
    assert f8.off_rc_scale - f8.off_rc_codes == 256 * 128 * 64 * 128
    f4 = bd.ssm_layout_query(cfg(readcopy=bd.SSM_RC_FP4_B16))
    assert f4.off_rc_scale - f4.off_rc_codes == 256 * 128 * 64 * 64
    assert f4.off_rc_tscale - f4.off_rc_scale == 256 * 128 * 64 * 8


@pytest.mark.parametrize("P,N", [(16, 16), (16, 128), (32, 16), (32, 128), (64, 16), (64, 128)])
def test_every_accepted_mamba2_shape(P, N):
    lay = bd.ssm_layout_query(cfg(dim_p=P, dim_n=N))
    assert lay.off_ring[0] >= 256 * 128 * P * N * 4


@pytest.mark.parametrize("kw,status", [
    (dict(kind=5), bd.SSM_E_ARG),
    (dict(in_dtype=7), bd.SSM_E_ARG),
    (dict(readcopy=3), bd.SSM_E_ARG),
    (dict(heads=6, groups=4), bd.SSM_E_SHAPE),
    (dict(dim_p=48), bd.SSM_E_SHAPE),
    (dict(dim_p=128), bd.SSM_E_SHAPE),
    (dict(dim_n=8), bd.SSM_E_SHAPE),
    (dict(window=0), bd.SSM_E_SHAPE),
    (dict(window=33), bd.SSM_E_SHAPE),
    (dict(max_draft=0), bd.SSM_E_SHAPE),
    (dict(max_draft=9, window=16), bd.SSM_E_SHAPE),
    (dict(max_draft=5, window=4), bd.SSM_E_SHAPE),
    (dict(batch=-1), bd.SSM_E_SHAPE),
    (dict(batch=1, heads=1 << 21, groups=1 << 21, max_draft=8), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_GDN, batch=1, heads=1 << 22, groups=1 << 22, max_draft=4), bd.SSM_E_SHAPE),
    (dict(readcopy=bd.SSM_RC_FP8_ROW, dim_p=32, dim_n=64), bd.SSM_E_UNSUPPORTED),
    (dict(readcopy=bd.SSM_RC_FP8_ROW, dim_n=32), bd.SSM_E_UNSUPPORTED),
    (dict(readcopy=bd.SSM_RC_FP4_B16, dim_n=32), bd.SSM_E_UNSUPPORTED),
    (dict(dim_p=32, dim_n=4), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_GDN, groups=64), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_GDN, dim_p=32), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_GDN, window=32, max_draft=2), bd.SSM_E_UNSUPPORTED),
    (dict(kind=bd.SSM_KDA, groups=64), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_KDA, dim_p=32), bd.SSM_E_SHAPE),
    (dict(kind=bd.SSM_KDA, readcopy=bd.SSM_RC_FP8_ROW, dim_n=32), bd.SSM_E_SHAPE),
    (dict(kind=3), bd.SSM_E_ARG),
    (dict(share_ckpt=2), bd.SSM_E_ARG),
])
def test_bad_configs_rejected(kw, status):
    with pytest.raises(bd.SSMError) as ei:
        bd.ssm_layout_query(cfg(**kw))
    assert ei.value.status == status


def raw(fn, *args):
    return getattr(bd._lib, fn)(*args)


def empty_state(**kw):
    c = cfg(batch=0, **kw)
    st = bd.ssm_state()
    s = raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), ctypes.c_void_p(FAKE),
            1 << 40, None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None)
    assert s == bd.SSM_OK
    return st


def m2_in(addr=FAKE):
    return bd.ssm_m2_in(addr, addr, addr, addr)


def gdn_in(addr=FAKE):
    return bd.ssm_gdn_in(addr, addr, addr, addr, addr)


def test_init_validation():
    c = cfg()
    st = bd.ssm_state()
    v = ctypes.c_void_p
    assert raw("ssm_ckpt_init", None, ctypes.byref(c), v(FAKE), 1 << 40, None, v(FAKE),
               v(FAKE), None) == bd.SSM_E_ARG
    assert raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), None, 1 << 40, None, v(FAKE),
               v(FAKE), None) == bd.SSM_E_ARG
    assert raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), v(FAKE), 1024, None, v(FAKE),
               v(FAKE), None) == bd.SSM_E_ARG  # too small
    assert raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), v(FAKE + 16), 1 << 40, None,
               v(FAKE), v(FAKE), None) == bd.SSM_E_ALIGN
    assert raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), v(FAKE), 1 << 40, v(FAKE + 4),
               v(FAKE), v(FAKE), None) == bd.SSM_E_ALIGN
    assert raw("ssm_ckpt_init", ctypes.byref(st), ctypes.byref(c), v(FAKE), 1 << 40, None,
               None, v(FAKE), None) == bd.SSM_E_ARG  # Mamba-2 needs A and D


def test_bad_magic_rejected():
    st = bd.ssm_state()
    y = ctypes.c_void_p(FAKE)
    assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_E_STATE
    assert raw("ssm_flush", ctypes.byref(st), 0, None) == bd.SSM_E_STATE
    assert raw("ssm_spec_rollback", ctypes.byref(st), y, None) == bd.SSM_E_STATE


def test_state_machine_errors_without_device():
    st = empty_state(max_draft=4)
    y = ctypes.c_void_p(FAKE)
    assert st.count_hi == 0 and st.pending == 0
    # rollback without drafts
    assert raw("ssm_spec_rollback", ctypes.byref(st), y, None) == bd.SSM_E_STATE
    # too many drafts
    assert raw("ssm_spec_append", ctypes.byref(st), 5, ctypes.byref(m2_in()), y, None) == \
        bd.SSM_E_CAPACITY
    assert raw("ssm_spec_append", ctypes.byref(st), 0, ctypes.byref(m2_in()), y, None) == bd.SSM_E_ARG
    # misaligned inputs / outputs
    assert raw("ssm_spec_append", ctypes.byref(st), 2, ctypes.byref(m2_in(FAKE + 2)), y, None) == \
        bd.SSM_E_ALIGN
    assert raw("ssm_spec_append", ctypes.byref(st), 2, ctypes.byref(m2_in()),
               ctypes.c_void_p(FAKE + 8), None) == bd.SSM_E_ALIGN
    assert raw("ssm_spec_append", ctypes.byref(st), 2, None, y, None) == bd.SSM_E_ARG
    # a valid append on an empty batch: drafts now pending
    assert raw("ssm_spec_append", ctypes.byref(st), 3, ctypes.byref(m2_in()), y, None) == bd.SSM_OK
    assert st.pending == 3
    assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_E_STATE
    assert raw("ssm_flush", ctypes.byref(st), 0, None) == bd.SSM_E_STATE
    assert raw("ssm_spec_append", ctypes.byref(st), 1, ctypes.byref(m2_in()), y, None) == bd.SSM_E_STATE
    assert raw("ssm_flush", ctypes.byref(st), 7, None) == bd.SSM_E_ARG
    assert raw("ssm_spec_rollback", ctypes.byref(st), None, None) == bd.SSM_E_ARG
    assert raw("ssm_spec_rollback", ctypes.byref(st), y, None) == bd.SSM_OK
    assert st.pending == 0 and st.count_hi == 3
    # decodes advance the host bound; the L-th folds
    for _ in range(12):
        assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_OK
    assert st.count_hi == 15
    assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_OK
    assert (st.count_lo, st.count_hi) == (0, 15)  # lo < L <= hi before the fold
    assert raw("ssm_flush", ctypes.byref(st), bd.SSM_FLUSH_ALL, None) == bd.SSM_OK
    assert (st.count_lo, st.count_hi) == (0, 0)


def test_capacity_bound_after_rollback():
    st = empty_state(max_draft=4, window=4)  # cap = 7
    y = ctypes.c_void_p(FAKE)
    for _ in range(3):
        assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_OK
    assert (st.count_lo, st.count_hi) == (3, 3)
    assert raw("ssm_spec_append", ctypes.byref(st), 4, ctypes.byref(m2_in()), y, None) == bd.SSM_OK
    assert raw("ssm_spec_rollback", ctypes.byref(st), y, None) == bd.SSM_OK
    # counts in [3, 7] before the automatic fold -> [0, 3] after it
    assert (st.count_lo, st.count_hi) == (0, 3)


def test_conventional_and_pack_validation():
    c = cfg()
    v = ctypes.c_void_p
    assert raw("ssm_conventional_step", ctypes.byref(c), None, ctypes.byref(m2_in()), v(FAKE),
               v(FAKE), v(FAKE), None) == bd.SSM_E_ARG
    assert raw("ssm_conventional_step", ctypes.byref(c), v(FAKE + 4), ctypes.byref(m2_in()),
               v(FAKE), v(FAKE), v(FAKE), None) == bd.SSM_E_ALIGN
    assert raw("ssm_conventional_step", ctypes.byref(c), v(FAKE), ctypes.byref(m2_in()), None,
               v(FAKE), v(FAKE), None) == bd.SSM_E_ARG
    bad = cfg(dim_p=48)
    assert raw("ssm_tiles_pack", ctypes.byref(bad), v(FAKE), v(FAKE), None) == bd.SSM_E_SHAPE
    assert raw("ssm_tiles_unpack", ctypes.byref(c), None, v(FAKE), None) == bd.SSM_E_ARG
    assert raw("ssm_debug_codec", 12, v(FAKE), v(FAKE), 4, None) == bd.SSM_E_ARG
    assert raw("ssm_debug_codec", -1, v(FAKE), v(FAKE), 4, None) == bd.SSM_E_ARG
    assert raw("ssm_debug_codec", 0, None, None, 0, None) == bd.SSM_OK  # empty: nothing to do


def test_snapshot_baseline_validation():
    c = cfg(max_draft=4)
    v = ctypes.c_void_p
    snap = lambda cc, nd, h=FAKE, s=FAKE, inp=m2_in(), y=FAKE: raw(
        "ssm_conventional_spec_snapshot", ctypes.byref(cc), v(h), v(s), nd, ctypes.byref(inp),
        v(FAKE), v(FAKE), v(y), None)
    assert snap(c, 0) == bd.SSM_E_CAPACITY
    assert snap(c, 9) == bd.SSM_E_CAPACITY
    assert snap(c, 2, h=FAKE + 4) == bd.SSM_E_ALIGN
    assert snap(c, 2, y=FAKE + 8) == bd.SSM_E_ALIGN
    assert snap(c, 2, inp=m2_in(FAKE + 2)) == bd.SSM_E_ALIGN
    assert snap(cfg(batch=0), 4) == bd.SSM_OK  # nothing to do
    # GDN / KDA: gdn inputs, A and D ignored (NULL allowed); the same validation otherwise
    for kind in (bd.SSM_GDN, bd.SSM_KDA):
        g = cfg(kind=kind, groups=128, max_draft=4)
        gsnap = lambda cc, nd, h=FAKE, inp=None: raw(
            "ssm_conventional_spec_snapshot", ctypes.byref(cc), v(h), v(FAKE), nd,
            ctypes.byref(inp if inp is not None else gdn_in()), None, None, v(FAKE), None)
        assert gsnap(g, 9) == bd.SSM_E_CAPACITY
        assert gsnap(g, 2, h=FAKE + 4) == bd.SSM_E_ALIGN
        assert gsnap(g, 2, inp=gdn_in(FAKE + 8)) == bd.SSM_E_ALIGN
        assert gsnap(cfg(kind=kind, groups=128, batch=0), 4) == bd.SSM_OK
        assert raw("ssm_conventional_spec_snapshot", ctypes.byref(g), v(FAKE), v(FAKE), 2, None,
                   None, None, v(FAKE), None) == bd.SSM_E_ARG
        assert raw("ssm_conventional_spec_select", ctypes.byref(cfg(kind=kind, groups=128, batch=0)),
                   v(FAKE), v(FAKE), 2, v(FAKE), None) == bd.SSM_OK
    assert raw("ssm_conventional_spec_snapshot", ctypes.byref(c), None, v(FAKE), 2,
               ctypes.byref(m2_in()), v(FAKE), v(FAKE), v(FAKE), None) == bd.SSM_E_ARG
    sel = lambda cc, nd, acc=FAKE: raw("ssm_conventional_spec_select", ctypes.byref(cc), v(FAKE),
                                       v(FAKE), nd, v(acc), None)
    assert sel(c, 0) == bd.SSM_E_CAPACITY
    assert sel(c, 2, acc=FAKE + 2) == bd.SSM_E_ALIGN
    assert raw("ssm_conventional_spec_select", ctypes.byref(c), v(FAKE), v(FAKE), 2, None,
               None) == bd.SSM_E_ARG
    assert sel(cfg(batch=0), 4) == bd.SSM_OK


def test_debug_flags_validation():
    out = ctypes.c_int32(0)
    assert raw("ssm_debug_flags", ctypes.byref(bd.ssm_state()), ctypes.byref(out), 0,
               None) == bd.SSM_E_STATE
    st = empty_state()
    assert raw("ssm_debug_flags", ctypes.byref(st), None, 0, None) == bd.SSM_E_ARG


def test_restore_and_fork_validation():
    v = ctypes.c_void_p
    I = lambda *xs: (ctypes.c_int32 * max(len(xs), 1))(*xs)
    assert raw("ssm_restore", ctypes.byref(bd.ssm_state()), v(FAKE), None) == bd.SSM_E_STATE
    assert raw("ssm_fork", ctypes.byref(bd.ssm_state()), I(0), I(1), 1, None) == bd.SSM_E_STATE
    st = empty_state(max_draft=4)
    assert raw("ssm_restore", ctypes.byref(st), None, None) == bd.SSM_E_ARG
    assert raw("ssm_restore", ctypes.byref(st), v(FAKE + 2), None) == bd.SSM_E_ALIGN
    for _ in range(3):
        assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), v(FAKE),
                   None) == bd.SSM_OK
    assert (st.count_lo, st.count_hi) == (3, 3)
    assert raw("ssm_restore", ctypes.byref(st), v(FAKE), None) == bd.SSM_OK  # empty batch
    assert (st.count_lo, st.count_hi) == (0, 3)  # device counts now unknown below the old bound
    assert raw("ssm_fork", ctypes.byref(st), I(), I(), 0, None) == bd.SSM_OK
    assert raw("ssm_fork", ctypes.byref(st), I(), I(), -1, None) == bd.SSM_E_ARG
    assert raw("ssm_fork", ctypes.byref(st), None, None, 1, None) == bd.SSM_E_ARG
    assert raw("ssm_fork", ctypes.byref(st), I(0), I(0), 1, None) == bd.SSM_E_ARG  # batch is 0
    # index checks on a batch of 4 (each case fails before any launch)
    st.cfg.batch = 4
    assert raw("ssm_fork", ctypes.byref(st), I(0, 1), I(2, 2), 2, None) == bd.SSM_E_ARG
    assert raw("ssm_fork", ctypes.byref(st), I(0, 2), I(2, 3), 2, None) == bd.SSM_E_ARG  # chain
    assert raw("ssm_fork", ctypes.byref(st), I(0), I(4), 1, None) == bd.SSM_E_ARG
    assert raw("ssm_fork", ctypes.byref(st), I(-1), I(1), 1, None) == bd.SSM_E_ARG
    st.cfg.batch = 0
    assert raw("ssm_spec_append", ctypes.byref(st), 2, ctypes.byref(m2_in()), v(FAKE),
               None) == bd.SSM_OK
    assert raw("ssm_restore", ctypes.byref(st), v(FAKE), None) == bd.SSM_E_STATE
    assert raw("ssm_fork", ctypes.byref(st), I(), I(), 0, None) == bd.SSM_E_STATE


def test_host_ring_start_follows_the_ring_model():
    """The host's copy of the ring start (used to launch without reading the device pointers)
    moves exactly as the oracle's ring model moves every sequence's start in lock step, and is
    dropped once the counts are known only on the device."""
    from oracle.ring import Ring

    for window, max_draft in ((16, 1), (4, 4), (5, 3)):
        st = empty_state(max_draft=max_draft, window=window)
        ring = Ring(cap=st.lay.ring_cap, L=window)
        y = ctypes.c_void_p(FAKE)
        assert st.ring_start == 0
        for t in range(3 * window + 2):
            assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_OK
            ring.decode()
            ring.flush_if_full()
            assert (st.ring_start, st.count_lo, st.count_hi) == (ring.start, ring.count, ring.count), t
        assert raw("ssm_flush", ctypes.byref(st), bd.SSM_FLUSH_ALL, None) == bd.SSM_OK
        ring.flush_all()
        assert (st.ring_start, st.count_hi) == (ring.start, 0)
        for _ in range(window - 1):
            assert raw("ssm_replay_decode", ctypes.byref(st), ctypes.byref(m2_in()), y, None) == bd.SSM_OK
            ring.decode()
        assert st.ring_start == ring.start
        # drafts keep the start (only a rollback makes the counts device-side)
        assert raw("ssm_spec_append", ctypes.byref(st), 1, ctypes.byref(m2_in()), y, None) == bd.SSM_OK
        assert st.ring_start == ring.start
        assert raw("ssm_spec_rollback", ctypes.byref(st), y, None) == bd.SSM_OK
        assert st.ring_start == -1
        # and it stays unknown: the launches read the device pointers from here on
        assert raw("ssm_flush", ctypes.byref(st), bd.SSM_FLUSH_ALL, None) == bd.SSM_OK
        assert st.ring_start == -1

    st = empty_state(window=4)
    assert raw("ssm_restore", ctypes.byref(st), ctypes.c_void_p(FAKE), None) == bd.SSM_OK
    assert st.ring_start == -1
    st = empty_state(window=4, share_ckpt=1)
    assert st.ring_start == -1  # shared checkpoints: the slot comes from the device


def test_stream_read_validation():
    v = ctypes.c_void_p
    sr = lambda src, nbytes, out, blocks: raw("ssm_debug_stream_read", v(src), ctypes.c_uint64(nbytes),
                                              v(out), blocks, None)
    assert sr(FAKE, 1 << 20, FAKE, 0) == bd.SSM_E_ARG          # no workgroups
    assert sr(FAKE, 1 << 20, FAKE, (1 << 20) + 1) == bd.SSM_E_ARG
    assert sr(FAKE, (1 << 20) + 8, FAKE, 64) == bd.SSM_E_ARG   # not whole 16-byte units
    assert sr(None, 1 << 20, FAKE, 64) == bd.SSM_E_ARG
    assert sr(FAKE + 8, 1 << 20, FAKE, 64) == bd.SSM_E_ALIGN
    assert sr(FAKE, 1 << 20, FAKE + 2, 64) == bd.SSM_E_ALIGN
    assert sr(FAKE, 0, FAKE, 64) == bd.SSM_OK                  # empty: nothing launched
