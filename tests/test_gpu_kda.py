"""GPU parity of the Kimi Delta Attention path (per-channel gated delta rule: backward-sweep
replay with an elementwise decay, UT/WY flush with a gated Gram matrix on MFMA, speculative
verify and rollback, conventional step) against the fp64 oracle's sequential KDA recurrence."""
import numpy as np
import pytest
import torch

import oracle
from harness import GdnTokens, assert_close, sample_pairs, to_dev
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


def kda_oracle(S0, tok, pairs, scale=1.0, snap_after=()):
    q, k, v, beta, g = tok.head_inputs(pairs)
    S0p = None if S0 is None else np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    return oracle.kda_sequential(S0p, q, k, v, beta, g, scale=scale, snap_after=snap_after)


def _kshape(B, H, dv, dk, L, bf16=True, S=1):
    return synth.Shape(synth.KDA, B, H, H, dv, dk, L, S, in_bf16=bf16)


def make(shape, seed, s0_std, scale=1.0):
    S0 = synth.initial_state(shape, seed, s0_std) if s0_std else None
    cfg = bd.make_config(bd.SSM_KDA, shape.batch, shape.heads, shape.heads, shape.dim_p,
                         shape.dim_n, shape.window, shape.max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, 0, scale)
    return bd.State(cfg, None if S0 is None else S0.to(DEV), None, None), S0, cfg


def run_kda(shape, seed, T, s0_std, pairs, scale=1.0):
    st, S0, _ = make(shape, seed, s0_std, scale)
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
    oo, _, osn = kda_oracle(S0, tok, pairs, scale, snaps)
    go = torch.stack(os_, 1).cpu().double().numpy()
    return go, (np.stack(cks, 1) if cks else None), oo, osn, st, S0, tok


@pytest.mark.parametrize("B,H,dv,dk,L,bf16,T,S", [
    (2, 3, 64, 64, 4, True, 21, 1),
    (1, 2, 128, 128, 16, False, 37, 1),
    (2, 2, 128, 64, 8, True, 19, 1),
    (1, 3, 64, 128, 32, True, 70, 1),      # more than 16 entries per call, two fold chunks
    (2, 2, 128, 128, 1, True, 5, 1),       # L = 1: every token through the fused fold
    (1, 2, 128, 128, 8, True, 75, 3),      # cap 10: lock-step windows start at every slot
])
def test_kda_decode_shapes(B, H, dv, dk, L, bf16, T, S):
    shape = _kshape(B, H, dv, dk, L, bf16, S)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    go, gck, oo, osn, st, *_ = run_kda(shape, 170 + T, T, 0.3162, pairs, scale=0.5 if L == 8 else 1.0)
    assert_close(go, oo, (-1,), "KDA replay outputs")
    if gck is not None:
        assert_close(gck, osn, (-2, -1), "KDA flushed checkpoints")
    c = st.cfg
    assert st.st.ring_start == (T // L) * L % st.layout.ring_cap
    p = st.region(st.layout.off_ptr, c.batch * c.heads * 16).view(torch.int32).view(c.batch, c.heads, 4).cpu()
    assert torch.all(p[..., 0] == st.st.ring_start) and torch.all(p[..., 1] == st.st.count_lo)


def test_kda_serving_batch_sampled_heads():
    w = synth.WORKLOADS["kda_b256"]
    shape = w["shape"]
    pairs = sample_pairs(shape.batch, shape.heads, 16)
    go, gck, oo, osn, *_ = run_kda(shape, w["seed"], 64, w["h0_std"], pairs)
    assert_close(go, oo, (-1,), "KDA replay outputs")
    assert_close(gck, osn, (-2, -1), "KDA flushed checkpoints")


def test_kda_flush_all_and_export():
    shape = _kshape(2, 3, 128, 128, 16)
    pairs = [(b, h) for b in range(2) for h in range(3)]
    st, S0, _ = make(shape, 181, 0.3)
    tok = GdnTokens(shape, 181)
    o = torch.empty(2, 3, 128, device=DEV)
    for t in range(11):  # a partial window
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), o)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    nat = torch.empty(2, 3, 128, 128, device=DEV)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    _, ST, _ = kda_oracle(S0, tok, pairs)
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "KDA state after flush-all")


@pytest.mark.parametrize("B,H,dv,dk,bf16", [(2, 3, 64, 128, False), (256, 32, 128, 128, True)])
def test_kda_conventional_step(B, H, dv, dk, bf16):
    shape = _kshape(B, H, dv, dk, 16, bf16)
    S0 = synth.initial_state(shape, 190, 0.3)
    cfg = bd.make_config(bd.SSM_KDA, B, H, H, dv, dk, 16, 1,
                         bd.SSM_IN_BF16 if bf16 else bd.SSM_IN_F32, 0, 0.8)
    tiles = torch.empty(B * H * dv * dk, device=DEV)
    bd.ssm_tiles_pack(cfg, S0.to(DEV).contiguous(), tiles)
    tok = GdnTokens(shape, 190)
    o = torch.empty(B, H, dv, device=DEV)
    pairs = sample_pairs(B, H, 12) if B * H > 12 else [(b, h) for b in range(B) for h in range(H)]
    outs = []
    for t in range(3):
        bd.ssm_conventional_step(cfg, tiles, to_dev(tok.draw(t), DEV), None, None, o)
        outs.append(o.clone())
    nat = torch.empty(B, H, dv, dk, device=DEV)
    bd.ssm_tiles_unpack(cfg, tiles, nat)
    torch.cuda.synchronize()
    oo, ST, _ = kda_oracle(S0, tok, pairs, 0.8)
    go = np.stack([np.stack([outs[t][b, h].cpu().double().numpy() for t in range(3)])
                   for (b, h) in pairs])
    assert_close(go, oo, (-1,), "KDA conventional outputs")
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "KDA conventional state")


@pytest.mark.parametrize("case", ["small", "odd", "wide", "long", "serving"])
def test_kda_spec_rounds_match_oracle(case):
    if case == "small":
        shape, seed, R, s0 = _kshape(2, 3, 64, 64, 4, False, 4), 151, 20, 0.3
    elif case == "odd":
        shape, seed, R, s0 = _kshape(3, 2, 128, 64, 8, True, 3), 152, 16, 0.3
    elif case == "wide":  # eight drafts: the eight-query verify
        shape, seed, R, s0 = _kshape(2, 3, 128, 128, 16, True, 8), 154, 16, 0.3
    elif case == "long":  # four drafts on a 24-entry window: calls that see 25..27 entries
        shape, seed, R, s0 = _kshape(2, 2, 128, 128, 24, True, 4), 155, 24, 0.3
    else:
        shape, seed, R, s0 = _kshape(256, 32, 128, 128, 16, True, 4), 153, 16, 0.3162
    S = shape.max_draft
    Bn, H, dv, dk = shape.batch, shape.heads, shape.dim_p, shape.dim_n
    pairs = sample_pairs(Bn, H, 16) if Bn * H > 64 else [(b, h) for b in range(Bn) for h in range(H)]
    st, S0, _ = make(shape, seed, s0, 0.75)
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
    oo, ST, _ = oracle.kda_spec_rounds(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"],
                                       acc, scale=0.75)
    assert_close(go, oo, (-1,), "KDA draft outputs")
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "KDA state after the speculative rounds")
