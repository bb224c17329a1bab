"""GPU checks of the speculative path (Mamba-2): draft outputs against the oracle, rollback that
moves pointers only (bitwise), and the state after speculative rounds equal, bit for bit, to the
state reached by decoding the accepted tokens one at a time.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import assert_close, sample_pairs, to_dev
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def make_state(shape, seed, h0_std):
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, h0_std) if h0_std else None
    cfg = bd.make_config(bd.SSM_MAMBA2, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, shape.window, shape.max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32)
    st = bd.State(cfg, None if h0 is None else h0.to(DEV), A.to(DEV), D.to(DEV))
    return st, A, D, h0


def regions(st):
    """Raw byte regions of a state: ckpt, ring x/B/dt, pointers (device tensors)."""
    c, L = st.cfg, st.layout
    esz = 2 if c.in_dtype == bd.SSM_IN_BF16 else 4
    cap = L.ring_cap
    B, H, G, P, N = c.batch, c.heads, c.groups, c.dim_p, c.dim_n
    return {
        "ckpt": st.region(L.off_ckpt, B * H * P * N * 4),
        "x": st.region(L.off_ring[0], B * H * cap * P * esz).view(B, H, cap, P * esz),
        "B": st.region(L.off_ring[1], B * G * cap * N * esz).view(B, G, cap, N * esz),
        "dt": st.region(L.off_ring[3], B * H * cap * 4).view(B, H, cap, 4),
        "ptr": st.region(L.off_ptr, B * H * 16).view(torch.int32).view(B, H, 4),
    }


def committed_ring(st, b_list=None):
    """Bytes of every committed ring entry, keyed by (b, h, entry index after the checkpoint)."""
    r = regions(st)
    ptr = r["ptr"].cpu()
    c = st.cfg
    hpg = c.heads // c.groups
    cap = st.layout.ring_cap
    out = {}
    xs, Bs, ds = r["x"].cpu(), r["B"].cpu(), r["dt"].cpu()
    for b in (b_list if b_list is not None else range(c.batch)):
        for h in range(c.heads):
            start, count = int(ptr[b, h, 0]), int(ptr[b, h, 1])
            for e in range(count):
                s = (start + e) % cap
                out[(b, h, e)] = (bytes(xs[b, h, s].numpy()), bytes(Bs[b, h // hpg, s].numpy()),
                                  bytes(ds[b, h, s].numpy()))
    return out


def run_spec(shape, seed, R, S, pairs, h0_std):
    st, A, D, h0 = make_state(shape, seed, h0_std)
    ys, acc_all, drafts, tiles = [], [], [], []
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    y = torch.empty(shape.batch, S, shape.heads, shape.dim_p, device=DEV)
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), y)
        ys.append(y[bi, :, hi].clone())
        acc = synth.accept_counts(shape.batch, S, 1002, r)
        acc_all.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
    torch.cuda.synchronize()
    return st, A, D, h0, torch.stack(ys, 1).cpu().double().numpy(), torch.stack(acc_all, 1), drafts


def oracle_spec(A, D, h0, drafts, acc, pairs, shape, S):
    hpg = shape.heads // shape.groups
    x = np.stack([np.stack([synth.to_f64(d["x"][b, :, h]) for d in drafts]) for (b, h) in pairs])
    Bm = np.stack([np.stack([synth.to_f64(d["B"][b, :, h // hpg]) for d in drafts]) for (b, h) in pairs])
    Cm = np.stack([np.stack([synth.to_f64(d["C"][b, :, h // hpg]) for d in drafts]) for (b, h) in pairs])
    dt = np.stack([np.stack([synth.to_f64(d["dt"][b, :, h]) for d in drafts]) for (b, h) in pairs])
    accp = np.stack([acc[b].numpy() for (b, _) in pairs]).astype(np.int32)
    L = shape.window
    snaps = []
    for i in range(len(pairs)):
        tot = int(accp[i].sum())
        snaps.append(list(range(L, tot + 1, L)))
    ns = max(1, max(len(s) for s in snaps))
    snap_arr = np.full((len(pairs), ns), -1, dtype=np.int32)
    for i, s in enumerate(snaps):
        snap_arr[i, :len(s)] = s
    hs = np.array([h for (_, h) in pairs])
    h0p = None if h0 is None else np.stack([h0[b, h].double().numpy() for (b, h) in pairs])
    y, hT, sn = oracle.m2_spec_rounds(A.double().numpy()[hs], D.double().numpy()[hs], h0p, x, Bm,
                                      Cm, dt, accp, snap_after=snap_arr)
    return y, hT, sn, accp


@pytest.mark.parametrize("case", ["small", "odd", "six", "wide", "serving"])
def test_spec_rounds_match_oracle(case):
    if case == "small":
        w = synth.WORKLOADS["m2_small"]
        shape, seed, R, h0s = w["shape"], 0, 40, 0.0
    elif case == "odd":
        shape = synth.Shape(synth.MAMBA2, 3, 6, 3, 64, 64, 8, 3, in_bf16=True)
        seed, R, h0s = 21, 30, 0.3
    elif case == "six":  # six drafts: the eight-query verify with two unused queries, P = 32
        shape = synth.Shape(synth.MAMBA2, 2, 5, 5, 32, 64, 8, 6, in_bf16=True)
        seed, R, h0s = 22, 20, 0.3
    elif case == "wide":  # eight drafts over a 32-entry window: up to 39 entries per call
        shape = synth.Shape(synth.MAMBA2, 3, 4, 2, 64, 128, 32, 8, in_bf16=True)
        seed, R, h0s = 23, 24, 0.3
    else:
        w = synth.WORKLOADS["m2_b256_spec"]
        shape, seed, R, h0s = w["shape"], w["seed"], w["rounds"], w["h0_std"]
    S = shape.max_draft
    pairs = (sample_pairs(shape.batch, shape.heads, 16) if shape.batch * shape.heads > 64
             else [(b, h) for b in range(shape.batch) for h in range(shape.heads)])
    st, A, D, h0, gy, acc, drafts = run_spec(shape, seed, R, S, pairs, h0s)
    oy, hT, sn, accp = oracle_spec(A, D, h0, drafts, acc, pairs, shape, S)
    assert_close(gy, oy, (-1,), "draft outputs")
    # checkpoint after the last round: position L * floor(total / L) for each sequence
    L = shape.window
    nat = torch.empty(shape.batch, shape.heads, shape.dim_p, shape.dim_n, device=DEV)
    bd.ssm_ckpt_export(st, nat)
    ptr = regions(st)["ptr"].cpu()
    torch.cuda.synchronize()
    for i, (b, h) in enumerate(pairs):
        tot = int(accp[i].sum())
        nf = tot // L
        assert int(ptr[b, h, 1]) == tot - nf * L
        if nf:
            assert_close(nat[b, h].cpu().double().numpy(), sn[i, nf - 1], (-2, -1),
                         "checkpoint of (%d,%d) after %d folds" % (b, h, nf))


def test_rollback_zero_is_bitwise_noop():
    shape = synth.Shape(synth.MAMBA2, 4, 8, 4, 64, 128, 16, 4, in_bf16=True)
    st, A, D, h0 = make_state(shape, 31, 0.3)
    y1 = torch.empty(4, 8, 64, device=DEV)
    for t in range(7):
        bd.ssm_replay_decode(st, to_dev(synth.token_inputs(shape, 31, "decode", t), DEV), y1)
    torch.cuda.synchronize()
    before = {k: v.clone() for k, v in regions(st).items() if k in ("ckpt", "ptr")}
    ring_before = committed_ring(st)
    y = torch.empty(4, 4, 8, 64, device=DEV)
    bd.ssm_spec_append(st, 4, to_dev(synth.token_inputs(shape, 31, "draft", 0, ntok=4), DEV), y)
    bd.ssm_spec_rollback(st, torch.zeros(4, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert bd.ssm_debug_flags(st) == 0
    after = regions(st)
    assert torch.equal(before["ckpt"], after["ckpt"])
    assert torch.equal(before["ptr"], after["ptr"])
    assert committed_ring(st) == ring_before
    # negative / oversized accept counts are clamped to [0, pending]
    bd.ssm_spec_append(st, 2, to_dev(synth.token_inputs(shape, 31, "draft", 1, ntok=2), DEV),
                       y[:, :2].contiguous())
    bd.ssm_spec_rollback(st, torch.tensor([-3, 0, 9, 1], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    cnt = regions(st)["ptr"].cpu()[..., 1]
    assert cnt[0].eq(7).all() and cnt[1].eq(7).all() and cnt[2].eq(9).all() and cnt[3].eq(8).all()
    # the clamp is recorded in the flag word, which reading with clear=True resets
    assert bd.ssm_debug_flags(st, clear=True) == bd.SSM_FLAG_ACCEPT_CLAMPED
    assert bd.ssm_debug_flags(st) == 0


@pytest.mark.parametrize("case", ["small", "odd", "serving"])
def test_snapshot_baseline_matches_oracle(case):
    """Conventional speculation (per-draft snapshots, then the accepted one restored) computes
    the same draft outputs and final state as the oracle's speculative rounds."""
    if case == "small":
        w = synth.WORKLOADS["m2_small"]
        shape, seed, R, h0s = w["shape"], 0, 12, 0.0
    elif case == "odd":
        shape = synth.Shape(synth.MAMBA2, 3, 6, 3, 32, 16, 8, 3, in_bf16=True)
        seed, R, h0s = 22, 10, 0.3
    else:
        w = synth.WORKLOADS["m2_b256_spec"]
        shape, seed, R, h0s = w["shape"], w["seed"], 6, w["h0_std"]
    S = shape.max_draft
    Bn, H, P, N = shape.batch, shape.heads, shape.dim_p, shape.dim_n
    pairs = (sample_pairs(Bn, H, 16) if Bn * H > 64 else [(b, h) for b in range(Bn) for h in range(H)])
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, h0s) if h0s else None
    cfg = bd.make_config(bd.SSM_MAMBA2, Bn, H, shape.groups, P, N, shape.window, S,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32)
    h = torch.empty(Bn * H * P * N, device=DEV)
    if h0 is None:
        h.zero_()
    else:
        bd.ssm_tiles_pack(cfg, h0.to(DEV), h)
    snap = torch.empty(S, Bn * H * P * N, device=DEV)
    y = torch.empty(Bn, S, H, P, device=DEV)
    Ad, Dd = A.to(DEV), D.to(DEV)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([hh for (_, hh) in pairs], device=DEV)
    ys, accs, drafts = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_conventional_spec_snapshot(cfg, h, snap, S, to_dev(d, DEV), Ad, Dd, y)
        ys.append(y[bi, :, hi].clone())
        acc = synth.accept_counts(Bn, S, 1002, r)
        accs.append(acc)
        if r == 0:  # the restore moves exactly the accepted snapshot (bitwise)
            before = h.clone()
        bd.ssm_conventional_spec_select(cfg, h, snap, S, acc.to(DEV))
        if r == 0:
            torch.cuda.synchronize()
            hv, bv, sv = h.view(Bn, -1), before.view(Bn, -1), snap.view(S, Bn, -1)
            for b in range(Bn):
                a = int(acc[b])
                assert torch.equal(hv[b], sv[a - 1, b] if a > 0 else bv[b]), b
    torch.cuda.synchronize()
    gy = torch.stack(ys, 1).cpu().double().numpy()
    oy, hT, _, _ = oracle_spec(A, D, h0, drafts, torch.stack(accs, 1), pairs, shape, S)
    assert_close(gy, oy, (-1,), "snapshot-baseline draft outputs")
    nat = torch.empty(Bn, H, P, N, device=DEV)
    bd.ssm_tiles_unpack(cfg, h, nat)
    torch.cuda.synchronize()
    got = np.stack([nat[b, hh].cpu().double().numpy() for (b, hh) in pairs])
    assert_close(got, hT, (-2, -1), "state after the snapshot rounds")


def test_spec_state_equals_sequential_decode_bitwise():
    """After speculative rounds, each sequence's checkpoint, pointers and committed ring entries
    equal, bit for bit, those of a one-sequence state that decoded only its accepted tokens
    (same flush points, same fold kernel, ring entries are copies of the input bits)."""
    shape = synth.Shape(synth.MAMBA2, 3, 4, 2, 64, 128, 8, 4, in_bf16=True)
    seed, R, S = 41, 25, 4
    st, A, D, h0 = make_state(shape, seed, 0.3)
    y = torch.empty(shape.batch, S, shape.heads, shape.dim_p, device=DEV)
    drafts, accs = [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), y)
        acc = synth.accept_counts(shape.batch, S, 1002, r)
        accs.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
    torch.cuda.synchronize()
    spec_r = regions(st)
    P, N, H = shape.dim_p, shape.dim_n, shape.heads
    ck = spec_r["ckpt"].view(torch.float32).view(shape.batch, H * P * N)
    for b in range(shape.batch):
        # same ring capacity as the speculative state, so the slots line up too
        cfg = bd.make_config(bd.SSM_MAMBA2, 1, H, shape.groups, P, N, shape.window, S,
                             bd.SSM_IN_BF16)
        sb = bd.State(cfg, h0[b:b + 1].contiguous().to(DEV), A.to(DEV), D.to(DEV))
        y1 = torch.empty(1, H, P, device=DEV)
        for r in range(R):
            for j in range(int(accs[r][b])):
                tok = {k: v[b:b + 1, j:j + 1].contiguous() for k, v in drafts[r].items()}
                bd.ssm_replay_decode(sb, to_dev(tok, DEV), y1)
        torch.cuda.synchronize()
        seq_r = regions(sb)
        assert torch.equal(seq_r["ckpt"].view(torch.float32).view(-1), ck[b]), b
        assert torch.equal(seq_r["ptr"][0][..., :2], spec_r["ptr"][b][..., :2]), b
        ring_seq = committed_ring(sb)
        ring_spec = {(0, h, e): v for (bb, h, e), v in committed_ring(st, [b]).items()}
        assert ring_seq == ring_spec, b


@pytest.mark.parametrize("rc", [0, 2])
def test_draft_outputs_ignore_later_drafts(rc):
    """Draft j's output depends on the committed entries and drafts 1..j only (news, para 3:
    drafts are appended to the buffer and verified in one pass). With NaN in every input of the
    last draft, the earlier drafts' outputs are bit-identical to those of a run with finite
    inputs there: the entries a query does not see are selected away, not multiplied by zero."""
    shape = synth.Shape(synth.MAMBA2, 4, 8, 4, 64, 128, 16, 4, in_bf16=True)
    S = shape.max_draft
    outs = []
    for poison in (False, True):
        A, D = synth.head_constants(shape, 41)
        h0 = synth.initial_state(shape, 41, 0.3)
        cfg = bd.make_config(bd.SSM_MAMBA2, 4, 8, 4, 64, 128, 16, S, bd.SSM_IN_BF16, rc)
        st = bd.State(cfg, h0.to(DEV), A.to(DEV), D.to(DEV))
        y1 = torch.empty(4, 8, 64, device=DEV)
        for t in range(5):
            bd.ssm_replay_decode(st, to_dev(synth.token_inputs(shape, 41, "decode", t), DEV), y1)
        d = synth.token_inputs(shape, 41, "draft", 0, ntok=S)
        if poison:
            for key in ("x", "B", "C", "dt"):
                d[key][:, S - 1] = float("nan")
        y = torch.empty(4, S, 8, 64, device=DEV)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), y)
        torch.cuda.synchronize()
        outs.append(y.cpu())
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0][:, :S - 1], outs[1][:, :S - 1])
    assert torch.isnan(outs[1][:, S - 1]).all()
