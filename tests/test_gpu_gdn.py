"""GPU parity of the Gated DeltaNet replay path (backward-sweep replay, UT/WY flush on MFMA,
speculative verify and rollback, conventional step) against the fp64 oracle's sequential gated
delta rule."""
import numpy as np
import pytest
import torch

import oracle
from harness import GdnTokens, assert_close, gdn_oracle, sample_pairs, to_dev
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def tiles_of(st, pairs):
    c = st.cfg
    P, N = c.dim_p, c.dim_n
    ck = st.region(st.layout.off_ckpt, c.batch * c.heads * P * N * 4).view(torch.float32)
    ck = ck.view(c.batch * c.heads, N // 4, P, 4)
    idx = torch.tensor([b * c.heads + h for (b, h) in pairs], device=DEV)
    return ck.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N).cpu().double().numpy()


def run_gdn(shape, seed, T, s0_std, pairs, scale=1.0):
    S0 = synth.initial_state(shape, seed, s0_std) if s0_std else None
    cfg = bd.make_config(bd.SSM_GDN, shape.batch, shape.heads, shape.heads, shape.dim_p,
                         shape.dim_n, shape.window, shape.max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, 0, scale)
    st = bd.State(cfg, None if S0 is None else S0.to(DEV), None, None)
    tok = GdnTokens(shape, seed)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    os_, cks = [], []
    L = shape.window
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), o)
        os_.append(o[bi, hi].clone())
        if (t + 1) % L == 0:
            cks.append(tiles_of(st, pairs))
    torch.cuda.synchronize()
    snaps = list(range(L, T + 1, L))
    oo, _, osn = gdn_oracle(S0, tok, pairs, scale, snaps)
    go = torch.stack(os_, 1).cpu().double().numpy()
    return go, (np.stack(cks, 1) if cks else None), oo, osn, st, S0, tok


def _gshape(B, H, dv, dk, L, bf16=True, S=1):
    return synth.Shape(synth.GDN, B, H, H, dv, dk, L, S, in_bf16=bf16)


def check_lockstep_pointers(st, T, L):
    """Lock step: the start and count the launches took from the host are the device's."""
    c = st.cfg
    assert st.st.ring_start == (T // L) * L % st.layout.ring_cap
    p = st.region(st.layout.off_ptr, c.batch * c.heads * 16).view(torch.int32)
    p = p.view(c.batch, c.heads, 4).cpu()
    assert torch.all(p[..., 0] == st.st.ring_start) and torch.all(p[..., 1] == st.st.count_lo)


@pytest.mark.parametrize("B,H,dv,dk,L,bf16,T,S", [
    (2, 3, 64, 64, 4, True, 21, 1),
    (1, 2, 128, 128, 16, False, 37, 1),
    (2, 2, 128, 64, 8, True, 19, 1),
    (1, 3, 64, 128, 32, True, 70, 1),
    (2, 2, 128, 128, 1, True, 5, 1),
    (2, 2, 128, 128, 16, True, 150, 4),  # cap 19: lock-step windows start at every slot in turn
])
def test_gdn_decode_shapes(B, H, dv, dk, L, bf16, T, S):
    shape = _gshape(B, H, dv, dk, L, bf16, S)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    go, gck, oo, osn, st, *_ = run_gdn(shape, 70 + T, T, 0.3162, pairs, scale=0.5 if L == 8 else 1.0)
    assert_close(go, oo, (-1,), "GDN replay outputs")
    if gck is not None:
        assert_close(gck, osn, (-2, -1), "GDN flushed checkpoints")
    check_lockstep_pointers(st, T, L)


def test_gdn_serving_batch_sampled_heads():
    w = synth.WORKLOADS["gdn_b256"]
    shape = w["shape"]
    pairs = sample_pairs(shape.batch, shape.heads, 24)
    go, gck, oo, osn, *_ = run_gdn(shape, w["seed"], w["steps"], w["h0_std"], pairs)
    assert_close(go, oo, (-1,), "GDN replay outputs")
    assert_close(gck, osn, (-2, -1), "GDN flushed checkpoints")


def test_gdn_flush_all_and_export():
    shape = _gshape(2, 2, 128, 128, 16)
    pairs = [(b, h) for b in range(2) for h in range(2)]
    go, gck, oo, osn, st, S0, tok = run_gdn(shape, 81, 21, 0.3162, pairs)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    out = torch.empty(2, 2, 128, 128, device=DEV)
    bd.ssm_ckpt_export(st, out)
    torch.cuda.synchronize()
    _, ST, _ = gdn_oracle(S0, tok, pairs)
    assert_close(out.cpu().double().numpy().reshape(4, 128, 128), ST, (-2, -1),
                 "GDN checkpoint after flush(ALL) of 5 entries")


@pytest.mark.parametrize("B,H,dv,dk,bf16", [(2, 3, 64, 128, False), (256, 32, 128, 128, True)])
def test_gdn_conventional_step(B, H, dv, dk, bf16):
    shape = _gshape(B, H, dv, dk, 16, bf16)
    S0 = synth.initial_state(shape, 90, 0.3162)
    cfg = bd.make_config(bd.SSM_GDN, B, H, H, dv, dk, 16, 1,
                         bd.SSM_IN_BF16 if bf16 else bd.SSM_IN_F32)
    tiles = torch.empty(B * H * dv * dk, device=DEV)
    bd.ssm_tiles_pack(cfg, S0.to(DEV).contiguous(), tiles)
    pairs = sample_pairs(B, H, 16) if B * H > 64 else [(b, h) for b in range(B) for h in range(H)]
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    tok = GdnTokens(shape, 90)
    o = torch.empty(B, H, dv, device=DEV)
    os_ = []
    for t in range(7):
        bd.ssm_conventional_step(cfg, tiles, to_dev(tok.draw(t), DEV), None, None, o)
        os_.append(o[bi, hi].clone())
    nat = torch.empty(B, H, dv, dk, device=DEV)
    bd.ssm_tiles_unpack(cfg, tiles, nat)
    torch.cuda.synchronize()
    oo, ST, _ = gdn_oracle(S0, tok, pairs)
    assert_close(torch.stack(os_, 1).cpu().double().numpy(), oo, (-1,), "GDN conventional outputs")
    assert_close(nat[bi, hi].cpu().double().numpy(), ST, (-2, -1), "GDN conventional state")


@pytest.mark.parametrize("case", ["small", "odd", "wide", "long", "serving"])
def test_gdn_spec_rounds_match_oracle(case):
    """Speculative rounds (drafts appended and verified in one pass, U{0..S} accepted, pointer
    rollback, fold when a sequence reaches L) against the oracle's speculative rounds."""
    if case == "small":
        shape, seed, R, s0 = synth.Shape(synth.GDN, 2, 3, 3, 64, 64, 4, 4, in_bf16=False), 51, 20, 0.3
    elif case == "odd":
        shape, seed, R, s0 = synth.Shape(synth.GDN, 3, 2, 2, 128, 64, 8, 3, in_bf16=True), 52, 16, 0.3
    elif case == "wide":  # eight drafts: the eight-query verify, up to 23 entries per call
        shape, seed, R, s0 = synth.Shape(synth.GDN, 2, 3, 3, 128, 128, 16, 8, in_bf16=True), 53, 16, 0.3
    elif case == "long":  # four drafts on a 24-entry window: calls that see 25..27 entries
        shape, seed, R, s0 = synth.Shape(synth.GDN, 2, 2, 2, 128, 128, 24, 4, in_bf16=True), 54, 24, 0.3
    else:
        w = synth.WORKLOADS["gdn_b256_spec"]
        shape, seed, R, s0 = w["shape"], w["seed"], 24, w["h0_std"]
    S = shape.max_draft
    Bn, H, dv, dk, L = shape.batch, shape.heads, shape.dim_p, shape.dim_n, shape.window
    pairs = sample_pairs(Bn, H, 16) if Bn * H > 64 else [(b, h) for b in range(Bn) for h in range(H)]
    S0 = synth.initial_state(shape, seed, s0)
    cfg = bd.make_config(bd.SSM_GDN, Bn, H, H, dv, dk, L, S,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, 0, 0.75)
    st = bd.State(cfg, S0.to(DEV), None, None)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(Bn, S, H, dv, device=DEV)
    outs, drafts, accs = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), o)
        outs.append(o[bi, :, hi].clone())
        acc = synth.accept_counts(Bn, S, 1002, r)
        accs.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
    nat = torch.empty(Bn, H, dv, dk, device=DEV)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    go = torch.stack(outs, 1).cpu().double().numpy()
    ins = {key: np.stack([np.stack([synth.to_f64(d[key][b, :, h]) for d in drafts])
                          for (b, h) in pairs]) for key in ("q", "k", "v", "beta", "g")}
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    oo, ST, _ = oracle.gdn_spec_rounds(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"],
                                       acc, scale=0.75)
    assert_close(go, oo, (-1,), "GDN draft outputs")
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "GDN state after the speculative rounds")


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA])
@pytest.mark.parametrize("case", ["small", "odd", "wide", "serving"])
def test_gdn_snapshot_baseline_matches_oracle(kind, case):
    """Conventional speculation for GDN and KDA (the state after every draft written as a
    snapshot, then each sequence's accepted one restored) computes the same draft outputs and
    final state as the oracle's speculative rounds; the restore moves exactly the accepted
    snapshot (bitwise)."""
    if case == "small":
        shape, seed, R = synth.Shape(kind, 2, 3, 3, 64, 64, 4, 4, in_bf16=False), 61, 12
    elif case == "odd":
        shape, seed, R = synth.Shape(kind, 3, 2, 2, 128, 64, 8, 3), 62, 10
    elif case == "wide":  # eight drafts: the eight-token snapshot kernel
        shape, seed, R = synth.Shape(kind, 2, 3, 3, 128, 128, 16, 8), 63, 6
    else:
        shape, seed, R = synth.Shape(kind, 256, 32, 32, 128, 128, 16, 4), 64, 6
    S = shape.max_draft
    Bn, H, dv, dk = shape.batch, shape.heads, shape.dim_p, shape.dim_n
    pairs = sample_pairs(Bn, H, 16) if Bn * H > 64 else [(b, h) for b in range(Bn) for h in range(H)]
    S0 = synth.initial_state(shape, seed, 0.3)
    cfg = bd.make_config(kind, Bn, H, H, dv, dk, shape.window, S,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, 0, 0.75)
    h = torch.empty(Bn * H * dv * dk, device=DEV)
    bd.ssm_tiles_pack(cfg, S0.to(DEV).contiguous(), h)
    snap = torch.empty(S, Bn * H * dv * dk, device=DEV)
    o = torch.empty(Bn, S, H, dv, device=DEV)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([hh for (_, hh) in pairs], device=DEV)
    outs, accs, drafts = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_conventional_spec_snapshot(cfg, h, snap, S, to_dev(d, DEV), None, None, o)
        outs.append(o[bi, :, hi].clone())
        acc = synth.accept_counts(Bn, S, 1002, r)
        accs.append(acc)
        if r == 0:
            before = h.clone()
        bd.ssm_conventional_spec_select(cfg, h, snap, S, acc.to(DEV))
        if r == 0:
            torch.cuda.synchronize()
            hv, bv, sv = h.view(Bn, -1), before.view(Bn, -1), snap.view(S, Bn, -1)
            for b in range(Bn):
                a = int(acc[b])
                assert torch.equal(hv[b], sv[a - 1, b] if a > 0 else bv[b]), b
    nat = torch.empty(Bn, H, dv, dk, device=DEV)
    bd.ssm_tiles_unpack(cfg, h, nat)
    torch.cuda.synchronize()
    go = torch.stack(outs, 1).cpu().double().numpy()
    ins = {key: np.stack([np.stack([synth.to_f64(d[key][b, :, hh]) for d in drafts])
                          for (b, hh) in pairs]) for key in ("q", "k", "v", "beta", "g")}
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    S0p = np.stack([S0[b, hh].double().numpy() for (b, hh) in pairs])
    spec = oracle.kda_spec_rounds if kind == synth.KDA else oracle.gdn_spec_rounds
    oo, ST, _ = spec(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"], acc, scale=0.75)
    assert_close(go, oo, (-1,), "snapshot-baseline draft outputs")
    got = np.stack([nat[b, hh].cpu().double().numpy() for (b, hh) in pairs])
    assert_close(got, ST, (-2, -1), "state after the snapshot rounds")


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA])
@pytest.mark.parametrize("rc", [0, 2])
def test_gdn_draft_outputs_ignore_later_drafts(kind, rc):
    """As for Mamba-2: with NaN in every input of the last draft, the earlier drafts' outputs
    (GDN and KDA verify, fp32 state or fp4 read copy) are bit-identical to those of a run with
    finite inputs there. An entry a query does not see contributes no coefficient and no value
    row to that query."""
    shape = synth.Shape(kind, 2, 3, 3, 128, 128, 16, 4, in_bf16=True)
    S = shape.max_draft
    outs = []
    for poison in (False, True):
        S0 = synth.initial_state(shape, 61, 0.3)
        cfg = bd.make_config(bd.SSM_GDN if kind == synth.GDN else bd.SSM_KDA, 2, 3, 3, 128, 128,
                             16, S, bd.SSM_IN_BF16, rc, 0.75)
        st = bd.State(cfg, S0.to(DEV), None, None)
        o1 = torch.empty(2, 3, 128, device=DEV)
        for t in range(5):
            bd.ssm_replay_decode(st, to_dev(synth.token_inputs(shape, 61, "decode", t), DEV), o1)
        d = synth.token_inputs(shape, 61, "draft", 0, ntok=S)
        if poison:
            for key in ("q", "k", "v", "beta", "g"):
                d[key][:, S - 1] = float("nan")
        o = torch.empty(2, S, 3, 128, device=DEV)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), o)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0][:, :S - 1], outs[1][:, :S - 1])
    assert torch.isnan(outs[1][:, S - 1]).all()
