"""GPU parity of the Mamba-2 replay path against the fp64 oracle, through the C ABI.

Every case draws seeded inputs (ssm_decode_state_amd.synth), runs decode steps on the GPU, and
compares every replay output and every checkpoint written by a flush with the sequential
recurrence of the oracle on the same input bits (tolerance: tests/harness.py).
"""
import numpy as np
import pytest
import torch

from harness import M2Tokens, assert_close, m2_oracle, sample_pairs, to_dev
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def tiles_of(state: "bd.State", pairs):
    """Checkpoint tiles of the given (b, h) pairs, natural [n][P][N] layout, read from device
    memory through the documented tile layout."""
    c = state.cfg
    P, N = c.dim_p, c.dim_n
    nbytes = c.batch * c.heads * P * N * 4
    ck = state.region(state.layout.off_ckpt, nbytes).view(torch.float32)
    ck = ck.view(c.batch * c.heads, N // 4, P, 4)
    idx = torch.tensor([b * c.heads + h for (b, h) in pairs], device=ck.device)
    t = ck.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N)
    return t.cpu().double().numpy()


def pointers(state: "bd.State"):
    c = state.cfg
    p = state.region(state.layout.off_ptr, c.batch * c.heads * 16).view(torch.int32)
    return p.view(c.batch, c.heads, 4).cpu()


def run_decode(shape, seed, steps, h0_std, pairs, rc=0, check_ckpt=True):
    """Decode `steps` tokens on the GPU; returns (gpu y [n][T][P], gpu ckpts [n][F][P][N],
    oracle y, oracle ckpts, tokens)."""
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, h0_std) if h0_std else None
    cfg = bd.make_config(bd.SSM_MAMBA2, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, shape.window, shape.max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc)
    Ad, Dd = A.to(DEV), D.to(DEV)
    st = bd.State(cfg, None if h0 is None else h0.to(DEV), Ad, Dd)
    tok = M2Tokens(shape, seed)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    ys, cks = [], []
    y = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    L = shape.window
    for t in range(steps):
        inp = to_dev(tok.draw(t), DEV)
        bd.ssm_replay_decode(st.st, inp, y)
        ys.append(y[bi, hi].clone())
        if check_ckpt and (t + 1) % L == 0:
            cks.append(tiles_of(st, pairs))
    torch.cuda.synchronize()
    gy = torch.stack(ys, 1).cpu().double().numpy()
    snaps = list(range(L, steps + 1, L)) if check_ckpt else []
    oy, _, osn = m2_oracle(A, D, h0, tok, pairs, snap_after=snaps)
    gck = np.stack(cks, 1) if cks else None
    return gy, gck, oy, osn, st


def _shape(B, H, G, P, N, L, bf16, S=1):
    return synth.Shape(synth.MAMBA2, B, H, G, P, N, L, S, in_bf16=bf16)


def test_small_workload_every_output_and_checkpoint():
    w = synth.WORKLOADS["m2_small"]
    shape = w["shape"]
    pairs = [(b, h) for b in range(shape.batch) for h in range(shape.heads)]
    gy, gck, oy, osn, st = run_decode(shape, w["seed"], w["steps"], w["h0_std"], pairs)
    assert_close(gy, oy, (-1,), "replay outputs")
    assert gck.shape[1] == w["steps"] // shape.window
    assert_close(gck, osn, (-2, -1), "flushed checkpoints")
    p = pointers(st)
    assert torch.all(p[..., 1] == 0) and torch.all(p[..., 0] == (w["steps"] % st.layout.ring_cap))


@pytest.mark.parametrize("B,H,G,P,N,L,bf16,T,S", [
    (3, 6, 3, 64, 128, 16, True, 37, 1),    # ragged head blocks, B/C shared by pairs of heads
    (2, 5, 5, 32, 64, 8, False, 19, 1),
    (1, 4, 2, 16, 128, 5, True, 13, 1),
    (2, 8, 8, 64, 16, 1, False, 5, 1),      # L = 1: every token is folded at once
    (2, 4, 1, 64, 64, 32, True, 70, 1),     # L = 32, one B/C group for all heads
    (1, 3, 3, 64, 32, 7, True, 22, 1),
    (2, 6, 3, 32, 16, 4, True, 11, 1),      # two row copies per wave, one quad per lane
    # rings with draft room (cap = L + S - 1): lock-step windows start at every slot in turn
    (2, 4, 4, 64, 128, 16, True, 150, 4),
    (1, 3, 3, 64, 32, 7, True, 60, 3),
])
def test_decode_shapes(B, H, G, P, N, L, bf16, T, S):
    shape = _shape(B, H, G, P, N, L, bf16, S)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    gy, gck, oy, osn, st = run_decode(shape, 11 + T, T, 0.3, pairs)
    assert_close(gy, oy, (-1,), "replay outputs")
    if gck is not None:
        assert_close(gck, osn, (-2, -1), "flushed checkpoints")
    # lock step: the start and count the launches took from the host are the device's
    cap = st.layout.ring_cap
    assert st.st.ring_start == (T // L) * L % cap
    p = pointers(st)
    assert torch.all(p[..., 0] == st.st.ring_start) and torch.all(p[..., 1] == st.st.count_lo)


@pytest.mark.parametrize("B,H", [(4, 128), (5, 103)])
def test_decode_at_the_launch_geometry_switch(B, H):
    """Serving head dimensions (P=64, N=128, L=16, bf16) on both sides of the launch geometry
    switch: 512 heads run one head per workgroup, 515 (a ragged last workgroup) four. Every
    output and flushed checkpoint against the oracle."""
    shape = _shape(B, H, H, 64, 128, 16, True)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    gy, gck, oy, osn, _ = run_decode(shape, 900 + B, 34, 0.3162, pairs)
    assert_close(gy, oy, (-1,), "replay outputs")
    assert_close(gck, osn, (-2, -1), "flushed checkpoints")


def test_serving_batch_sampled_heads():
    """The serving-batch workload at full size (B=256, H=128, P=64, N=128, L=16, bf16 inputs,
    256 steps) in the launch configuration the benchmark times; outputs and flushed checkpoints
    of a sample of heads checked against the oracle."""
    w = synth.WORKLOADS["m2_b256"]
    shape = w["shape"]
    pairs = sample_pairs(shape.batch, shape.heads, 24)
    gy, gck, oy, osn, _ = run_decode(shape, w["seed"], w["steps"], w["h0_std"], pairs)
    assert_close(gy, oy, (-1,), "replay outputs")
    assert_close(gck, osn, (-2, -1), "flushed checkpoints")


def test_flush_all_and_export():
    shape = _shape(2, 4, 4, 64, 64, 8, True)
    A, D = synth.head_constants(shape, 5)
    h0 = synth.initial_state(shape, 5, 0.3)
    cfg = bd.make_config(bd.SSM_MAMBA2, 2, 4, 4, 64, 64, 8, 1, bd.SSM_IN_BF16)
    st = bd.State(cfg, h0.to(DEV), A.to(DEV), D.to(DEV))
    out = torch.empty(2, 4, 64, 64, device=DEV)
    bd.ssm_ckpt_export(st.st, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), h0)  # pack/unpack round trip is exact
    tok = M2Tokens(shape, 5)
    y = torch.empty(2, 4, 64, device=DEV)
    for t in range(11):  # one fold at 8, three entries left
        bd.ssm_replay_decode(st.st, to_dev(tok.draw(t), DEV), y)
    bd.ssm_flush(st.st, bd.SSM_FLUSH_ALL)
    bd.ssm_ckpt_export(st.st, out)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(2) for h in range(4)]
    _, hT, _ = m2_oracle(A, D, h0, tok, pairs)
    g = out.cpu().double().numpy().reshape(8, 64, 64)
    assert_close(g, hT, (-2, -1), "checkpoint after flush(ALL)")
    p = pointers(st)
    assert torch.all(p[..., 1] == 0) and torch.all(p[..., 0] == 11 % 8)
    # decoding goes on from the moved start (the launches take it from the host in lock step)
    assert st.st.ring_start == 11 % 8
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    ys = []
    for t in range(11, 24):  # a fold at 8 more entries, five left
        bd.ssm_replay_decode(st.st, to_dev(tok.draw(t), DEV), y)
        ys.append(y[bi, hi].clone())
    torch.cuda.synchronize()
    oy, _, _ = m2_oracle(A, D, h0, tok, pairs)
    assert_close(torch.stack(ys, 1).cpu().double().numpy(), oy[:, 11:], (-1,),
                 "replay outputs after flush(ALL)")
    p = pointers(st)
    assert st.st.count_lo == st.st.count_hi == 5
    assert torch.all(p[..., 0] == st.st.ring_start) and torch.all(p[..., 1] == 5)


@pytest.mark.parametrize("B,H,G,P,N,bf16", [(2, 4, 4, 16, 16, False), (3, 6, 2, 64, 128, True),
                                            (2, 5, 5, 32, 16, True),
                                            (4, 128, 128, 64, 128, True),   # 512 heads: one per workgroup
                                            (5, 103, 103, 64, 128, True),   # 515: four, ragged
                                            (256, 128, 128, 64, 128, True)])
def test_conventional_step(B, H, G, P, N, bf16):
    shape = _shape(B, H, G, P, N, 16, bf16)
    A, D = synth.head_constants(shape, 7)
    h0 = synth.initial_state(shape, 7, 0.3)
    cfg = bd.make_config(bd.SSM_MAMBA2, B, H, G, P, N, 16, 1,
                         bd.SSM_IN_BF16 if bf16 else bd.SSM_IN_F32)
    tiles = torch.empty(B * H * P * N, device=DEV)
    bd.ssm_tiles_pack(cfg, h0.to(DEV).contiguous(), tiles)
    Ad, Dd = A.to(DEV), D.to(DEV)
    pairs = sample_pairs(B, H, 16) if B * H > 64 else [(b, h) for b in range(B) for h in range(H)]
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    tok = M2Tokens(shape, 7)
    y = torch.empty(B, H, P, device=DEV)
    ys = []
    T = 9
    for t in range(T):
        bd.ssm_conventional_step(cfg, tiles, to_dev(tok.draw(t), DEV), Ad, Dd, y)
        ys.append(y[bi, hi].clone())
    nat = torch.empty(B, H, P, N, device=DEV)
    bd.ssm_tiles_unpack(cfg, tiles, nat)
    torch.cuda.synchronize()
    oy, hT, _ = m2_oracle(A, D, h0, tok, pairs)
    assert_close(torch.stack(ys, 1).cpu().double().numpy(), oy, (-1,), "conventional outputs")
    g = nat[bi, hi].cpu().double().numpy()
    assert_close(g, hT, (-2, -1), "conventional state")


def test_empty_batch_is_a_noop():
    cfg = bd.make_config(bd.SSM_MAMBA2, 0, 4, 4, 64, 64, 8, 2, bd.SSM_IN_BF16)
    A = torch.zeros(4, device=DEV)
    st = bd.State(cfg, None, A, A)
    z = torch.zeros(16, device=DEV)
    inp = {"x": z, "B": z, "C": z, "dt": z}
    for _ in range(9):
        bd.ssm_replay_decode(st.st, inp, z)
    bd.ssm_spec_append(st.st, 2, inp, z)
    bd.ssm_spec_rollback(st.st, torch.zeros(1, dtype=torch.int32, device=DEV))
    bd.ssm_flush(st.st, bd.SSM_FLUSH_ALL)
    torch.cuda.synchronize()


def test_codecs_match_format_definitions():
    from oracle import quant
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    finite = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    out = torch.empty(finite.numel(), device=DEV)
    bd.ssm_debug_codec(1, finite.to(DEV), out)
    np.testing.assert_array_equal(out.cpu().numpy(), quant.e4m3_decode(finite.numpy()))
    c4 = torch.arange(16, dtype=torch.uint8)
    out4 = torch.empty(16, device=DEV)
    bd.ssm_debug_codec(3, c4.to(DEV), out4)
    np.testing.assert_array_equal(out4.cpu().numpy(), quant.e2m1_decode(c4.numpy()))
    rng = np.random.default_rng(0)
    mags = quant.E4M3[:0x7F]
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([rng.standard_normal(50000) * 40, rng.standard_normal(5000) * 0.01,
                        mids, -mids, mags, [500.0, 1e30, -1e30, 0.0, -0.0, 1e-40]]).astype(np.float32)
    enc = torch.empty(v.size, dtype=torch.uint8, device=DEV)
    bd.ssm_debug_codec(0, torch.from_numpy(v).to(DEV), enc)
    np.testing.assert_array_equal(enc.cpu().numpy(), quant.e4m3_encode(v))
    m2 = quant.E2M1[:8]
    v2 = np.concatenate([rng.standard_normal(20000) * 3, (m2[1:] + m2[:-1]) / 2,
                         -(m2[1:] + m2[:-1]) / 2, m2, [7.0, 100.0, -0.0]]).astype(np.float32)
    enc2 = torch.empty(v2.size, dtype=torch.uint8, device=DEV)
    bd.ssm_debug_codec(2, torch.from_numpy(v2).to(DEV), enc2)
    np.testing.assert_array_equal(enc2.cpu().numpy(), quant.e2m1_encode(v2))
    del codes


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_hardware_conversions_match_format_definitions(fmt):
    """The gfx950 conversion instructions against the OCP definitions: decode of every code, and
    encode (after clamping to the largest magnitude) of random values, exact midpoints (ties to
    even), subnormals and saturating values."""
    from oracle import quant
    rng = np.random.default_rng(3)
    if fmt == "e4m3":
        codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
        dec_op, enc_op, table, top = 5, 4, quant.E4M3, 0x7E
        enc, dec = quant.e4m3_encode, quant.e4m3_decode
        scale = 40.0
    else:
        codes = np.arange(16, dtype=np.uint8)
        dec_op, enc_op, table, top = 7, 6, quant.E2M1, 0x7
        enc, dec = quant.e2m1_encode, quant.e2m1_decode
        scale = 3.0
    out = torch.empty(codes.size, device=DEV)
    bd.ssm_debug_codec(dec_op, torch.from_numpy(codes).to(DEV), out)
    np.testing.assert_array_equal(out.cpu().numpy(), dec(codes))
    mags = table[:top + 1]
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([rng.standard_normal(50000) * scale, mids, -mids, mags, -mags,
                        [1e9, -1e9, 0.0, -0.0]]).astype(np.float32)
    got = torch.empty(v.size, dtype=torch.uint8, device=DEV)
    bd.ssm_debug_codec(enc_op, torch.from_numpy(v).to(DEV), got)
    np.testing.assert_array_equal(got.cpu().numpy(), enc(v))


def test_packed_word_codecs_match_format_definitions():
    """The packed-word helpers the read-copy kernels use: every byte / nibble position decodes
    and encodes like the OCP definitions (byte i / nibble i = element i, low nibble first)."""
    from oracle import quant
    rng = np.random.default_rng(4)
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    c8 = rng.choice(fin, size=4 * 4096).astype(np.uint8)
    out = torch.empty(c8.size, device=DEV)
    bd.ssm_debug_codec(8, torch.from_numpy(c8.view(np.uint32).copy()).to(DEV), out)
    np.testing.assert_array_equal(out.cpu().numpy(), quant.e4m3_decode(c8))
    c4 = rng.integers(0, 16, size=8 * 4096).astype(np.uint8)
    words = (c4[0::2] | (c4[1::2] << 4)).astype(np.uint8).view(np.uint32).copy()
    out4 = torch.empty(c4.size, device=DEV)
    bd.ssm_debug_codec(9, torch.from_numpy(words).to(DEV), out4)
    np.testing.assert_array_equal(out4.cpu().numpy(), quant.e2m1_decode(c4))
    mags = quant.E4M3[:0x7F]
    v = np.concatenate([rng.standard_normal(4 * 8000) * 60, (mags[1:] + mags[:-1]) / 2,
                        -(mags[1:] + mags[:-1]) / 2, [1e9, -1e9, -0.0, 0.0, 3e-5, -600.0]])
    v = v[: v.size // 4 * 4].astype(np.float32)
    enc = torch.empty(v.size // 4, dtype=torch.int32, device=DEV)
    bd.ssm_debug_codec(10, torch.from_numpy(v).to(DEV), enc)
    np.testing.assert_array_equal(enc.cpu().numpy().view(np.uint8), quant.e4m3_encode(v))
    m2 = quant.E2M1[:8]
    v2 = np.concatenate([rng.standard_normal(8 * 8000) * 3, (m2[1:] + m2[:-1]) / 2,
                         -(m2[1:] + m2[:-1]) / 2, [1e9, -1e9, -0.0, 7.0, -0.1, 0.2]])
    v2 = v2[: v2.size // 8 * 8].astype(np.float32)
    enc2 = torch.empty(v2.size // 8, dtype=torch.int32, device=DEV)
    bd.ssm_debug_codec(11, torch.from_numpy(v2).to(DEV), enc2)
    b = enc2.cpu().numpy().view(np.uint8)
    got = np.empty(v2.size, dtype=np.uint8)
    got[0::2] = b & 0xF
    got[1::2] = b >> 4
    np.testing.assert_array_equal(got, quant.e2m1_encode(v2))


@pytest.mark.parametrize("nbytes,blocks", [(1 << 20, 64), ((1 << 20) + 16 * 37, 7), (16 * 5, 3)])
def test_stream_read_reads_every_unit_once(nbytes, blocks):
    """The streaming-read reference touches every 16-byte unit exactly once: the XOR of its
    per-wave outputs equals the XOR of every word of the input (ragged sizes and tails too)."""
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV)
    out = torch.zeros(4 * blocks, dtype=torch.int32, device=DEV)
    bd.ssm_debug_stream_read(src, out, blocks)
    torch.cuda.synchronize()
    exp = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == exp
