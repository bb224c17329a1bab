"""GPU checks of the low-precision read copy on Gated DeltaNet and Kimi Delta Attention layers
(dv x dk state tiles).

The copy is written from the fp32 state at init and at every flush and read only by the output
path (replay and speculative verify); the recurrence never sees it. Checks:
  * at init the copy's codes and scales equal, bit for bit, the oracle's fp32 emulation of the
    quantizer applied to the same initial state;
  * in the first window every output equals the oracle's replay form evaluated on the decoded
    copy (the only difference from the exact output is the copy itself);
  * every output stays within a closed-form bound around the exact (fp64, unquantized) output:
    |o - o_exact| <= scale * ||bound of row p||_2 * ||q||_2, because the replayed query r is q
    mapped through alpha_i (I - beta_i k_i k_i^T) with alpha, beta in (0, 1] and unit keys, so
    ||r||_2 <= ||q||_2 (1% slack for the bf16 rounding of the unit keys); with KDA's per-channel
    decay diag(alpha_i) in place of the scalar every factor still has norm <= 1;
  * every flushed fp32 state still matches the oracle to 1e-4, and the error does not drift;
  * speculative rounds through the read-copy verify stay within the same bound.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import GdnTokens, assert_close, sample_pairs, to_dev
from oracle import quant
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def copy_of(st, pairs, rc):
    """Codes / scales of the given heads in natural [n][dv][dk] / [n][dv][dk/16] order."""
    c, L = st.cfg, st.layout
    B, H, P, N = c.batch, c.heads, c.dim_p, c.dim_n
    idx = torch.tensor([b * H + h for (b, h) in pairs], device=DEV)
    if rc == bd.SSM_RC_FP8_ROW:
        codes = st.region(L.off_rc_codes, B * H * P * N).view(B * H, N // 16, P, 16)
        codes = codes.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N)
        s = st.region(L.off_rc_scale, B * H * P * 4).view(torch.float32).view(B * H, P)
        return codes.cpu().numpy(), s.index_select(0, idx).cpu().numpy()
    packed = st.region(L.off_rc_codes, B * H * P * N // 2).view(B * H, N // 32, P, 16)
    packed = packed.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N // 2)
    packed = packed.cpu().numpy()
    codes = np.empty((len(pairs), P, N), dtype=np.uint8)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    sb = st.region(L.off_rc_scale, B * H * P * (N // 16)).view(B * H, P, N // 16)
    ts = st.region(L.off_rc_tscale, B * H * 4).view(torch.float32)
    return codes, sb.index_select(0, idx).cpu().numpy(), ts.index_select(0, idx).cpu().numpy()


def emulate(S, rc):
    if rc == bd.SSM_RC_FP8_ROW:
        return quant.fp8_row_quantize(S)
    return quant.fp4_quantize(S)


def decoded_and_bound(S64, rc):
    """Oracle quantization of an fp64 state (cast to fp32): decoded copy and error bound."""
    S = S64.astype(np.float32)
    if rc == bd.SSM_RC_FP8_ROW:
        c, s = quant.fp8_row_quantize(S)
        return quant.fp8_row_decode(c, s), quant.fp8_row_bound(S, s)
    c, sb, st = quant.fp4_quantize(S)
    return quant.fp4_decode(c, sb, st), quant.fp4_bound(S, quant.fp4_scales(sb, st))


KINDS = [synth.GDN, synth.KDA]


def fns(kind):
    """The oracle's (sequential, replay-form, speculative-rounds) functions for the layer type."""
    if kind == synth.KDA:
        return oracle.kda_sequential, oracle.kda_replay_output, oracle.kda_spec_rounds
    return oracle.gdn_sequential, oracle.gdn_replay_output, oracle.gdn_spec_rounds


def make(shape, seed, rc, scale=1.0, max_draft=1):
    S0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(shape.kind, shape.batch, shape.heads, shape.heads, shape.dim_p,
                         shape.dim_n, shape.window, max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc, scale)
    return bd.State(cfg, S0.to(DEV), None, None), S0


def tiles_of(st, pairs):
    c = st.cfg
    P, N = c.dim_p, c.dim_n
    ck = st.region(st.layout.off_ckpt, c.batch * c.heads * P * N * 4).view(torch.float32)
    ck = ck.view(c.batch * c.heads, N // 4, P, 4)
    idx = torch.tensor([b * c.heads + h for (b, h) in pairs], device=DEV)
    return ck.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N).cpu().double().numpy()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("B,H,dv,dk", [(2, 3, 64, 64), (2, 2, 128, 128), (1, 3, 128, 64)])
def test_gdn_init_copy_is_bit_exact(rc, B, H, dv, dk, kind):
    shape = synth.Shape(kind, B, H, H, dv, dk, 8, 1)
    st, S0 = make(shape, 80 + dv + dk, rc)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    torch.cuda.synchronize()
    got = copy_of(st, pairs, rc)
    exp = emulate(np.stack([S0[b, h].numpy() for (b, h) in pairs]), rc)
    for g, e in zip(got, exp):
        np.testing.assert_array_equal(np.asarray(g), np.asarray(e))


def _bound(bnd, q, scale):
    """scale * ||row bound||_2 * ||q||_2 * 1.01 for every row: [n][dv]."""
    return abs(scale) * np.sqrt((bnd ** 2).sum(-1)) * np.linalg.norm(q, axis=-1)[:, None] * 1.01


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("case", ["small", "serving"])
def test_gdn_readcopy_decode(rc, case, kind):
    seq_fn, replay_fn, _ = fns(kind)
    if case == "small":
        shape = synth.Shape(kind, 2, 3, 3, 128, 128, 8, 1)
        seed, T, scale = 90 + rc + 7 * kind, 40, 0.5
        pairs = [(b, h) for b in range(2) for h in range(3)]
    else:
        w = synth.WORKLOADS["kda_b256" if kind == synth.KDA else "gdn_b256"]
        shape, seed, T, scale = w["shape"], w["seed"] + 10 * rc, 64, 1.0
        pairs = sample_pairs(shape.batch, shape.heads, 12)
    L = shape.window
    st, S0 = make(shape, seed, rc, scale)
    tok = GdnTokens(shape, seed)
    init_copy = copy_of(st, pairs, rc)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    os_, cks, copies = [], [], []
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), o)
        os_.append(o[bi, hi].clone())
        if (t + 1) % L == 0:
            cks.append(tiles_of(st, pairs))
            copies.append(copy_of(st, pairs, rc))
    torch.cuda.synchronize()
    go = torch.stack(os_, 1).cpu().double().numpy()
    snaps = list(range(L, T + 1, L))
    q, k, v, beta, g = tok.head_inputs(pairs)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    oo, _, osn = seq_fn(S0p, q, k, v, beta, g, scale=scale, snap_after=snaps)
    # (a) the fp32 recurrence is untouched by the copy
    assert_close(np.stack(cks, 1), osn, (-2, -1), "flushed fp32 states")
    # (b) first window: the oracle's replay form on the decoded initial copy
    S0n = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    if rc == bd.SSM_RC_FP8_ROW:
        dec0 = quant.fp8_row_decode(*init_copy)
    else:
        dec0 = quant.fp4_decode(*init_copy)
    for t in range(L):  # every token of the window replays from the initial copy
        exp = np.stack([replay_fn(dec0[i].astype(np.float64), q[i, t], k[i, :t + 1], v[i, :t + 1],
                                  beta[i, :t + 1], g[i, :t + 1], scale) for i in range(len(pairs))])
        assert_close(go[:, t], exp, (-1,), "first-window outputs on the decoded copy (t=%d)" % t)
    # (c) every output within the bound around the exact output; no drift across windows
    ratios = []
    for wdw in range(T // L):
        Sc = S0n if wdw == 0 else osn[:, wdw - 1]
        _, bnd = decoded_and_bound(Sc, rc)
        for j in range(L):  # the window's tokens replay from the copy of its start state
            t = wdw * L + j
            lim = _bound(bnd, q[:, t], scale)
            rms = np.sqrt((oo[:, t] ** 2).mean(axis=-1, keepdims=True))
            slack = 2e-4 * np.maximum(np.abs(oo[:, t]), rms)
            err = np.abs(go[:, t] - oo[:, t])
            assert np.all(err <= lim + slack), (wdw, j, float((err - lim - slack).max()))
            ratios.append(float((err / (lim + slack)).max()))
    per_window = np.array(ratios).reshape(T // L, L).max(axis=1)
    half = max(1, len(per_window) // 2)
    assert per_window[half:].max() <= 1.5 * per_window[:half].max() + 0.05, per_window
    # (d) the copy written at each flush is the quantization of the flushed state
    for wdw, cp in enumerate(copies):
        exp = emulate(osn[:, wdw].astype(np.float32), rc)
        mism = np.asarray(cp[0]) != np.asarray(exp[0])
        assert mism.mean() < 0.01, mism.mean()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
def test_gdn_readcopy_speculative_rounds(rc, kind):
    """Drafts verified through the read copy: every draft output within the bound around the
    exact output of the oracle's speculative rounds; the fp32 state exact."""
    _, _, spec_fn = fns(kind)
    shape = synth.Shape(kind, 2, 3, 3, 128, 128, 8, 4)
    seed, R, S = 95 + rc + 7 * kind, 10, 4
    st, S0 = make(shape, seed, rc, 1.0, max_draft=S)
    pairs = [(b, h) for b in range(2) for h in range(3)]
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(shape.batch, S, shape.heads, shape.dim_p, device=DEV)
    outs, drafts, accs = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), o)
        outs.append(o[bi, :, hi].clone())
        acc = synth.accept_counts(shape.batch, S, 1002, r)
        accs.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
    nat = torch.empty(shape.batch, shape.heads, shape.dim_p, shape.dim_n, device=DEV)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    go = torch.stack(outs, 1).cpu().double().numpy()
    ins = {key: np.stack([np.stack([synth.to_f64(d[key][b, :, h]) for d in drafts])
                          for (b, h) in pairs]) for key in ("q", "k", "v", "beta", "g")}
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    # the state each round's drafts were verified against, for the bound: the last folded one
    L = shape.window
    tot = np.cumsum(acc, axis=1)
    folds = [sorted(set(range(L, int(tot[i, -1]) + 1, L))) for i in range(len(pairs))]
    ns = max(1, max(len(f) for f in folds))
    snap = np.full((len(pairs), ns), -1, dtype=np.int32)
    for i, f in enumerate(folds):
        snap[i, :len(f)] = f
    oo, ST, sn = spec_fn(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"], acc, scale=1.0,
                         snap_after=snap)
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "fp32 state after the speculative rounds")
    for i in range(len(pairs)):
        committed = 0
        for r in range(R):
            nf = committed // L  # folds done before this round's drafts
            Sc = S0p[i] if nf == 0 else sn[i, nf - 1]
            _, bnd = decoded_and_bound(Sc[None], rc)
            for j in range(S):
                lim = _bound(bnd, ins["q"][i, r, j][None], 1.0)[0]
                rms = np.sqrt((oo[i, r, j] ** 2).mean())
                slack = 2e-4 * np.maximum(np.abs(oo[i, r, j]), rms)
                err = np.abs(go[i, r, j] - oo[i, r, j])
                assert np.all(err <= lim + slack), (i, r, j, float((err - lim - slack).max()))
            committed += int(acc[i, r])
