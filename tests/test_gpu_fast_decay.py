"""GPU parity of Gated DeltaNet and Kimi Delta Attention under gates that forget quickly.

A third of the decays are drawn as g = -U(10, 40) per token (synth.token_inputs(fast_decay=True)):
KDA key channels n % 3 == 0, GDN heads h % 3 == 0. Within one chunk of 16 entries such a channel's
cumulative log-decay falls by hundreds, far past fp32's exponent range (about -87 .. 88). The
flush's decay factors must therefore each stay <= 1 (exp of a difference of cumulative sums, never
a ratio, never a positive exponent): the KDA gated Gram matrix is formed over a binary split of the
chunk for that reason. Every output, every flushed state and the exported state after flush(ALL)
must match the fp64 oracle at 1e-4 and be finite; the same for speculative rounds (verify,
rollback, fold of a partial window), the conventional step and the read-copy fold.
"""
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

KINDS = [synth.GDN, synth.KDA]


def seq_fn(kind):
    return oracle.kda_sequential if kind == synth.KDA else oracle.gdn_sequential


def spec_fn(kind):
    return oracle.kda_spec_rounds if kind == synth.KDA else oracle.gdn_spec_rounds


def tiles_of(st, pairs):
    c = st.cfg
    P, N = c.dim_p, c.dim_n
    ck = st.region(st.layout.off_ckpt, c.batch * c.heads * P * N * 4).view(torch.float32)
    ck = ck.view(c.batch * c.heads, N // 4, P, 4)
    idx = torch.tensor([b * c.heads + h for (b, h) in pairs], device=DEV)
    return ck.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N).cpu().double().numpy()


def make(shape, seed, scale=1.0, rc=0):
    S0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(shape.kind, shape.batch, shape.heads, shape.heads, shape.dim_p,
                         shape.dim_n, shape.window, shape.max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc, scale)
    return bd.State(cfg, S0.to(DEV), None, None), S0


def finite(*arrays):
    for a in arrays:
        assert np.all(np.isfinite(a)), "non-finite values"


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,H,dv,dk,L,T,rc", [
    (2, 3, 128, 128, 16, 40, 0),   # serving head shape: fused window-closing folds, then 8 more
    (2, 3, 64, 64, 4, 21, 0),
    (1, 3, 64, 128, 32, 70, 0),    # two fold chunks per window
    (2, 3, 128, 64, 8, 30, 0),
    (2, 3, 128, 128, 16, 40, 1),   # read-copy fold (fp8) under the same gates
    (2, 3, 128, 128, 16, 40, 2),   # and fp4
])
def test_fast_decay_decode_and_flush_all(kind, B, H, dv, dk, L, T, rc):
    shape = synth.Shape(kind, B, H, H, dv, dk, L, 1)
    seed = 300 + T + 7 * kind + rc
    pairs = [(b, h) for b in range(B) for h in range(H)]
    st, S0 = make(shape, seed, 0.5 if L == 8 else 1.0, rc)
    scale = st.cfg.gdn_scale
    tok = GdnTokens(shape, seed, fast_decay=True)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(B, H, dv, device=DEV)
    os_, cks = [], []
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), o)
        os_.append(o[bi, hi].clone())
        if (t + 1) % L == 0:
            cks.append(tiles_of(st, pairs))
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)  # the partial last window
    nat = torch.empty(B, H, dv, dk, device=DEV)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    go = torch.stack(os_, 1).cpu().double().numpy()
    gck = np.stack(cks, 1)
    gend = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    finite(go, gck, gend)
    q, k, v, beta, g = tok.head_inputs(pairs)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    oo, ST, osn = seq_fn(kind)(S0p, q, k, v, beta, g, scale=scale,
                               snap_after=list(range(L, T + 1, L)))
    assert_close(gck, osn, (-2, -1), "flushed states, fast gates")
    assert_close(gend, ST, (-2, -1), "state after flush(ALL), fast gates")
    if rc == 0:  # (read-copy outputs are checked against their bound in the read-copy tests)
        assert_close(go, oo, (-1,), "replay outputs, fast gates")
    else:  # the window-closing steps emit from the new fp32 state, copy or not
        assert_close(go[:, L - 1::L], oo[:, L - 1::L], (-1,), "window-closing outputs, fast gates")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("case", ["small", "serving_heads"])
def test_fast_decay_spec_rounds(kind, case):
    if case == "small":
        shape, R = synth.Shape(kind, 2, 3, 3, 64, 64, 4, 3, in_bf16=False), 16
    else:
        shape, R = synth.Shape(kind, 3, 3, 3, 128, 128, 16, 4), 20
    seed = 320 + 7 * kind + R
    S = shape.max_draft
    Bn, H, dv, dk = shape.batch, shape.heads, shape.dim_p, shape.dim_n
    pairs = [(b, h) for b in range(Bn) for h in range(H)]
    st, S0 = make(shape, seed, 0.75)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(Bn, S, H, dv, device=DEV)
    outs, drafts, accs = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S, fast_decay=True)
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
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    finite(go, got)
    ins = {key: np.stack([np.stack([synth.to_f64(d[key][b, :, h]) for d in drafts])
                          for (b, h) in pairs]) for key in ("q", "k", "v", "beta", "g")}
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    oo, ST, _ = spec_fn(kind)(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"], acc,
                              scale=0.75)
    assert_close(go, oo, (-1,), "draft outputs, fast gates")
    assert_close(got, ST, (-2, -1), "state after the speculative rounds, fast gates")


@pytest.mark.parametrize("kind", KINDS)
def test_fast_decay_conventional_step(kind):
    B, H, dv, dk = 4, 6, 128, 128
    shape = synth.Shape(kind, B, H, H, dv, dk, 16, 1)
    S0 = synth.initial_state(shape, 340, 0.3162)
    cfg = bd.make_config(kind, B, H, H, dv, dk, 16, 1, bd.SSM_IN_BF16)
    tiles = torch.empty(B * H * dv * dk, device=DEV)
    bd.ssm_tiles_pack(cfg, S0.to(DEV).contiguous(), tiles)
    tok = GdnTokens(shape, 340, fast_decay=True)
    o = torch.empty(B, H, dv, device=DEV)
    pairs = sample_pairs(B, H, 12)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    outs = []
    for t in range(5):
        bd.ssm_conventional_step(cfg, tiles, to_dev(tok.draw(t), DEV), None, None, o)
        outs.append(o[bi, hi].clone())
    nat = torch.empty(B, H, dv, dk, device=DEV)
    bd.ssm_tiles_unpack(cfg, tiles, nat)
    torch.cuda.synchronize()
    q, k, v, beta, g = tok.head_inputs(pairs)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    oo, ST, _ = seq_fn(kind)(S0p, q, k, v, beta, g)
    go = torch.stack(outs, 1).cpu().double().numpy()
    got = nat[bi, hi].cpu().double().numpy()
    finite(go, got)
    assert_close(go, oo, (-1,), "conventional outputs, fast gates")
    assert_close(got, ST, (-2, -1), "conventional state, fast gates")
