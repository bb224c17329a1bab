"""The byte models behind bench.py's `achieved` rates, pinned to figures derived by hand from the
state layout and the input formats (no GPU needed).

Each model counts what one launch must move for one head: the state it reads (fp32 tile, or the
read copy), the buffered entries it reads, the call's inputs it reads, what it appends and what it
writes. The figures below are written out from the element sizes of the serving shapes (Mamba-2
P = 64, N = 128; GDN / KDA dv = dk = 128; bf16 inputs, fp32 dt / beta / g and outputs), not from
the functions under test, so a dropped or doubled term in a model fails here.
"""
import pytest

import bench

P, N = 64, 128          # Mamba-2 head: tile rows, state dim
DV = DK = 128           # GDN / KDA head
TILE_M2 = P * N * 4     # 32 768 B fp32 tile
TILE_GDN = DV * DK * 4  # 65 536 B


def test_mamba2_replay_model():
    entry = 128 + 256 + 4        # x (64 bf16), B (128 bf16), dt (fp32): one ring entry
    token = 128 + 256 + 256 + 4  # the token's x, B, C, dt read from the call's inputs
    y, count = 256, 4            # 64 fp32 outputs; the count written back
    for k in range(1, 17):
        want = TILE_M2 + (k - 1) * entry + token + entry + y + count
        assert bench.m2_replay_bytes_per_head(P, N, k) == want
    assert bench.m2_replay_bytes_per_head(P, N, 1) == 34060
    mean = sum(bench.m2_replay_bytes_per_head(P, N, k) for k in range(1, 16)) / 15
    assert mean == 36776  # the counts 1..15 the timed replay launches run at
    assert 256 * 128 * mean == 1205075968  # one launch at the serving batch


def test_mamba2_fold_conv_verify_models():
    entry, token = 388, 644
    # plain fold of L = 16 entries: tile read + written, the entries, the pointer entry
    assert bench.m2_flush_bytes_per_head(P, N, 16) == 2 * TILE_M2 + 16 * entry + 16 == 71760
    # the fused window-closing step as bench.py forms it: 15 buffered entries, the token, y
    fused = bench.m2_flush_bytes_per_head(P, N, 16) - entry + token + 256
    assert fused == 2 * TILE_M2 + 15 * entry + token + 256 + 16 == 72272
    assert bench.m2_conv_bytes_per_head(P, N) == 2 * TILE_M2 + token + 256 == 66436
    # verify of S = 4 drafts over kc committed entries: each draft read and appended, 4 outputs
    for kc in (0, 7, 15):
        assert bench.m2_verify_bytes_per_head(P, N, kc, 4) == \
            TILE_M2 + kc * entry + 4 * (token + entry) + 4 * 256 + 8
    # snapshot scheme: the state read once and written after each of the 4 drafts
    assert bench.m2_snapshot_bytes_per_head(P, N, 4) == 5 * TILE_M2 + 4 * token + 4 * 256


def test_read_copy_models():
    fp8 = P * N + P * 4              # one E4M3 byte per element + an fp32 scale per row
    fp4 = P * N // 2 + P * N // 16 + 4  # a nibble per element, an E4M3 scale per 16, one fp32
    assert (fp8, fp4) == (8448, 4612)
    for k in (1, 8, 15):
        plain = bench.m2_replay_bytes_per_head(P, N, k)
        assert bench.m2_rc_replay_bytes_per_head(P, N, k, 1) == plain - TILE_M2 + fp8
        assert bench.m2_rc_replay_bytes_per_head(P, N, k, 2) == plain - TILE_M2 + fp4
    g8 = DV * DK + DV * 4
    g4 = DV * DK // 2 + DV * DK // 16 + 4
    for k in (1, 8):
        plain = bench.gdn_replay_bytes_per_head(DV, DK, k)
        assert bench.gdn_rc_replay_bytes_per_head(DV, DK, k, 1) == plain - TILE_GDN + g8
        assert bench.gdn_rc_replay_bytes_per_head(DV, DK, k, 2) == plain - TILE_GDN + g4


@pytest.mark.parametrize("kda", [False, True])
def test_gdn_kda_models(kda):
    g = 4 * DK if kda else 4              # KDA: one fp32 log-decay per key channel
    entry = 256 + 256 + 4 + g             # k, v (bf16), beta, g
    token = 256 + 256 + 256 + 4 + g       # q, k, v, beta, g
    gsz = 4 * DK if kda else 4
    want8 = TILE_GDN + 7 * entry + token + entry + 512 + 4
    assert bench.gdn_replay_bytes_per_head(DV, DK, 8, gsz=gsz) == want8 == (75560 if kda else 70988)
    assert bench.gdn_conv_bytes_per_head(DV, DK, gsz=gsz) == 2 * TILE_GDN + token + 512 == \
        (132868 if kda else 132360)
    assert bench.gdn_verify_bytes_per_head(DV, DK, 5, 4, gsz=gsz) == \
        TILE_GDN + 5 * entry + 4 * (token + entry) + 4 * 512 + 8
    assert bench.gdn_snapshot_bytes_per_head(DV, DK, 4, gsz=gsz) == 5 * TILE_GDN + 4 * token + 4 * 512


def test_fork_bytes_per_sequence():
    bd = pytest.importorskip("ssm_decode_state_amd.binding",
                             reason="libssm_replay.so not built (run __graft_entry__.build())")
    for share, want in ((0, 4990976), (1, 796672)):
        cfg = bd.make_config(bd.SSM_MAMBA2, 256, 128, 128, P, N, 16, 1, bd.SSM_IN_BF16, 0, 1.0, share)
        lay = bd.ssm_layout_query(cfg)
        cap = lay.ring_cap
        rings = 128 * cap * (128 + 256 + 4)  # x, B (one group per head here), dt
        tiles = 0 if share else 128 * TILE_M2
        assert bench.seq_state_bytes(cfg, lay) == 128 * 16 + tiles + rings == want


def test_read_ceiling_interpolation():
    rc = {"by_bytes": {str(64 << 20): {"gbs": 5000.0}, str(256 << 20): {"gbs": 6000.0},
                       str(1 << 30): {"gbs": 7000.0}}}
    assert bench.ceiling_at(rc, 1 << 20) == 5000.0       # below the smallest size
    assert bench.ceiling_at(rc, 64 << 20) == 5000.0
    assert bench.ceiling_at(rc, 128 << 20) == pytest.approx(5500.0)  # halfway in log2(bytes)
    assert bench.ceiling_at(rc, 512 << 20) == pytest.approx(6500.0)
    assert bench.ceiling_at(rc, 4 << 30) == 7000.0       # above the largest


def test_fused_window_closing_step_models():
    # Mamba-2: tile read + written, 15 buffered entries, the token, y, the pointer entry
    m2 = 2 * TILE_M2 + 15 * 388 + 644 + 256 + 16
    assert m2 == 72272
    assert bench.m2_fused_step_bytes_per_head(P, N, 16) == m2
    assert bench.m2_fused_step_bytes_per_head(P, N, 16, 1) == m2 + 8448  # fp8 copy rewritten
    assert bench.m2_fused_step_bytes_per_head(P, N, 16, 2) == m2 + 4612  # fp4 copy rewritten
    for kda in (False, True):
        g = 4 * DK if kda else 4
        entry, token = 256 + 256 + 4 + g, 256 * 3 + 4 + g
        gdn = 2 * TILE_GDN + 15 * entry + token + 512 + 16
        assert gdn == (148304 if kda else 140176)
        assert bench.gdn_fused_step_bytes_per_head(DV, DK, 16, gsz=g) == gdn
        assert bench.gdn_fused_step_bytes_per_head(DV, DK, 16, 1, gsz=g) == gdn + DV * DK + DV * 4
        assert bench.gdn_fused_step_bytes_per_head(DV, DK, 16, 2, gsz=g) == \
            gdn + DV * DK // 2 + DV * DK // 16 + 4
    r = bench.fold_step_rate(2e9, [0.5, 0.5])  # 2 GB in 0.5 ms
    assert r["fold_step_achieved_gbs"] == pytest.approx(4000.0)
    assert r["fold_step_frac"] == pytest.approx(0.5)
    assert bench.fold_step_rate(1.0, []) == {}
