"""GPU checks of the low-precision read copy on Gated DeltaNet and Kimi Delta Attention layers
(dv x dk state tiles).

The copy is written from the fp32 state at init and at every flush and read only by the output
path (replay and speculative verify); the recurrence never sees it (news article, para 4).
Checks, in every window (decode) and every round (speculation):
  * copy: codes and scales equal, bit for bit, the oracle's fp32 quantizer applied to the GPU's
    own fp32 state (at init: to the initial state);
  * outputs: every output equals, to 1e-4, the oracle's replay form evaluated on the GPU's
    decoded copy with exactly the entries the GPU replayed (for drafts: the committed entries
    since the last fold and drafts 1..j); the window-closing step of a lock-step decode folds in
    fp32, rewrites the copy and emits its output from the new fp32 state, so that output is
    compared with the exact one at 1e-4;
  * bound: every output is within
        |o - o_exact| <= |scale| sum_n (bound[p, n] + |S_gpu - S_exact|[p, n]) |r[n]| + 1e-4 m
    of the exact fp64 output, where r is the replayed query (oracle.replay_query: the checkpoint
    enters the output only as scale S_c r), bound the format's closed-form element bound on the
    GPU's fp32 state with its own scales, and m = max(|o_copy|, rms) the 1e-4 metric's floor;
  * fp32 recurrence: every flushed state matches the oracle to 1e-4;
  * no drift: the least-squares slope of the per-window worst err / bound is not positive beyond
    three standard errors (printed, and appended to SSM_DRIFT_OUT when that names a file).
Adversarial initial tiles go through the same copy and output checks.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import (GdnTokens, TOL, adversarial_tiles, assert_close, assert_copy_exact, ckpt_of,
                     copy_of, decode_copy, drift_slope, elem_bound, report_drift, sample_pairs,
                     to_dev)
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")

KINDS = [synth.GDN, synth.KDA]


def fns(kind):
    """The oracle's (sequential, replay-form, speculative-rounds) functions for the layer type."""
    if kind == synth.KDA:
        return oracle.kda_sequential, oracle.kda_replay_output, oracle.kda_spec_rounds
    return oracle.gdn_sequential, oracle.gdn_replay_output, oracle.gdn_spec_rounds


def make(shape, seed, rc, scale=1.0, max_draft=1, S0=None):
    if S0 is None:
        S0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(shape.kind, shape.batch, shape.heads, shape.heads, shape.dim_p,
                         shape.dim_n, shape.window, max_draft,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc, scale)
    return bd.State(cfg, S0.to(DEV), None, None), S0


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("B,H,dv,dk", [(2, 3, 64, 64), (2, 2, 128, 128), (1, 3, 128, 64)])
def test_gdn_init_copy_is_bit_exact(rc, B, H, dv, dk, kind):
    shape = synth.Shape(kind, B, H, H, dv, dk, 8, 1)
    st, S0 = make(shape, 80 + dv + dk, rc)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    torch.cuda.synchronize()
    assert_copy_exact(np.stack([S0[b, h].numpy() for (b, h) in pairs]), copy_of(st, pairs, rc),
                      rc, "init copy")


def check_output(kind, scale, go, dec, Sg32, Se, rc_copy, rc, q, k, v, beta, g, exact, what):
    """One output vector per pair: 1e-4 against the oracle's replay on the decoded copy, and the
    bound around the exact output. Returns the worst err / bound."""
    _, replay_fn, _ = fns(kind)
    n = len(go)
    oc = np.stack([replay_fn(dec[i], q[i], k[i], v[i], beta[i], g[i], scale) for i in range(n)])
    assert_close(go, oc, (-1,), what + ": outputs on the decoded copy")
    r = np.stack([oracle.replay_query(q[i], k[i], v[i], beta[i], g[i], kind == synth.KDA)
                  for i in range(n)])
    lim_el = elem_bound(Sg32, rc_copy, rc) + np.abs(Sg32.astype(np.float64) - Se)
    lim = abs(scale) * np.einsum("ipn,in->ip", lim_el, np.abs(r))
    rms = np.sqrt((oc ** 2).mean(axis=-1, keepdims=True))
    slack = TOL * np.maximum(np.abs(oc), rms)
    err = np.abs(go - exact)
    assert np.all(err <= lim + slack), (what, float((err - lim - slack).max()))
    return float((err / (lim + slack)).max())


def run_decode(shape, seed, rc, T, scale, pairs, S0=None):
    seq_fn, _, _ = fns(shape.kind)
    L = shape.window
    st, S0 = make(shape, seed, rc, scale, S0=S0)
    tok = GdnTokens(shape, seed)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    torch.cuda.synchronize()
    cks, copies, os_ = [ckpt_of(st, pairs)], [copy_of(st, pairs, rc)], []
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), o)
        os_.append(o[bi, hi].clone())
        if (t + 1) % L == 0:
            cks.append(ckpt_of(st, pairs))
            copies.append(copy_of(st, pairs, rc))
    torch.cuda.synchronize()
    go = torch.stack(os_, 1).cpu().double().numpy()
    q, k, v, beta, g = tok.head_inputs(pairs)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    nwin = T // L
    oo, _, osn = seq_fn(S0p, q, k, v, beta, g, scale=scale, snap_after=list(range(L, T + 1, L)))
    if nwin:
        assert_close(np.stack(cks[1:nwin + 1], 1), osn, (-2, -1), "flushed fp32 states")
    for w, (Sg32, cp) in enumerate(zip(cks, copies)):
        assert_copy_exact(Sg32, cp, rc, "copy written at the start of window %d" % w)
    per_window = []
    for w in range((T + L - 1) // L):
        Sg32, cp = cks[w], copies[w]
        Se = S0p if w == 0 else osn[:, w - 1]
        dec = decode_copy(cp, rc)
        worst = 0.0
        for j in range(L):  # the window's tokens replay from the copy of its start state
            t = w * L + j
            if t >= T:
                break
            if j == L - 1:  # the fused window-closing step: output from the new fp32 state
                assert_close(go[:, t], oo[:, t], (-1,), "window-closing output (t=%d)" % t)
                continue
            e = slice(w * L, t + 1)
            worst = max(worst, check_output(shape.kind, scale, go[:, t], dec, Sg32, Se, cp, rc,
                                            q[:, t], k[:, e], v[:, e], beta[:, e], g[:, e],
                                            oo[:, t], "window %d token %d" % (w, j)))
        per_window.append(worst)
    return per_window


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("case", ["small", "small_f32", "serving"])
def test_gdn_readcopy_decode(rc, case, kind):
    if case.startswith("small"):  # small_f32: fp32 inputs
        shape = synth.Shape(kind, 2, 3, 3, 128, 128, 8, 1, in_bf16=case == "small")
        seed, T, scale = 90 + rc + 7 * kind + (5 if case == "small_f32" else 0), 64, 0.5
        pairs = [(b, h) for b in range(2) for h in range(3)]
    else:
        w = synth.WORKLOADS["kda_b256" if kind == synth.KDA else "gdn_b256"]
        shape, seed, T, scale = w["shape"], w["seed"] + 10 * rc, 512, 1.0  # 32 windows
        pairs = sample_pairs(shape.batch, shape.heads, 8)
    per_window = run_decode(shape, seed, rc, T, scale, pairs)
    slope, se = drift_slope(per_window)
    report_drift({"layer": "kda" if kind == synth.KDA else "gdn", "case": case,
                  "format": "fp8" if rc == 1 else "fp4", "windows": len(per_window),
                  "slope_per_window": slope, "stderr": se,
                  "mean_err_over_bound": float(np.mean(per_window)),
                  "max_err_over_bound": float(np.max(per_window))})
    assert slope <= 3 * se + 1e-9, (slope, se, per_window)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("dv,dk", [(128, 128), (64, 64)])
def test_gdn_adversarial_tiles(kind, rc, dv, dk):
    """Adversarial initial states: bit-exact copy at init and after the first fold, outputs on
    the decoded copy at 1e-4 and within the bound."""
    tiles = adversarial_tiles(dv, dk, 90 + dv + rc + 3 * kind)
    H = len(tiles)
    shape = synth.Shape(kind, 2, H, H, dv, dk, 8, 1)
    S0 = torch.from_numpy(np.stack([np.stack(tiles), np.stack(tiles[::-1])]))
    pairs = [(b, h) for b in range(2) for h in range(H)]
    per_window = run_decode(shape, 95 + dv + rc + 3 * kind, rc, 12, 1.0, pairs, S0=S0)
    assert len(per_window) == 2


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rc", [1, 2])
def test_gdn_readcopy_speculative_rounds(rc, kind):
    """Drafts verified through the read copy. After every round (rollback and any fold) the copy
    is bit-exact against the GPU's own state; every draft output equals the oracle's replay form
    on the decoded copy in effect for that round, with the committed entries since the last fold
    and drafts 1..j, and stays within the bound around the exact speculative output; the fp32
    state after the rounds is exact."""
    _, _, spec_fn = fns(kind)
    shape = synth.Shape(kind, 2, 3, 3, 128, 128, 8, 4)
    seed, R, S = 95 + rc + 7 * kind, 12, 4
    L = shape.window
    st, S0 = make(shape, seed, rc, 1.0, max_draft=S)
    pairs = [(b, h) for b in range(2) for h in range(3)]
    n = len(pairs)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    o = torch.empty(shape.batch, S, shape.heads, shape.dim_p, device=DEV)
    torch.cuda.synchronize()
    cks, copies = [ckpt_of(st, pairs)], [copy_of(st, pairs, rc)]  # before round r: index r
    outs, drafts, accs = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), o)
        outs.append(o[bi, :, hi].clone())
        acc = synth.accept_counts(shape.batch, S, 1002, r)
        accs.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
        cks.append(ckpt_of(st, pairs))
        copies.append(copy_of(st, pairs, rc))
    nat = torch.empty(shape.batch, shape.heads, shape.dim_p, shape.dim_n, device=DEV)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    for r, (Sg32, cp) in enumerate(zip(cks, copies)):
        assert_copy_exact(Sg32, cp, rc, "copy after round %d" % (r - 1))
    go = torch.stack(outs, 1).cpu().double().numpy()  # [n][R][S][dv]
    ins = {key: np.stack([np.stack([synth.to_f64(d[key][b, :, h]) for d in drafts])
                          for (b, h) in pairs]) for key in ("q", "k", "v", "beta", "g")}
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    S0p = np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    # exact states at every fold position (multiples of L of the committed count)
    tot = np.cumsum(acc, axis=1)
    folds = [list(range(L, int(tot[i, -1]) + 1, L)) for i in range(n)]
    ns = max(1, max(len(f) for f in folds))
    snap = np.full((n, ns), -1, dtype=np.int32)
    for i, f in enumerate(folds):
        snap[i, :len(f)] = f
    oo, ST, sn = spec_fn(S0p, ins["q"], ins["k"], ins["v"], ins["beta"], ins["g"], acc, scale=1.0,
                         snap_after=snap)
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, ST, (-2, -1), "fp32 state after the speculative rounds")
    for i in range(n):
        committed = {key: [] for key in ins}  # the accepted drafts, in order
        for r in range(R):
            c = len(committed["beta"])
            nf = c // L  # folds so far: one each time the committed count crossed a multiple of L
            Se = S0p[i] if nf == 0 else sn[i, nf - 1]
            Sg32, cp = cks[r][i:i + 1], tuple(x[i:i + 1] for x in copies[r])
            dec = decode_copy(cp, rc)
            for j in range(S):
                ent = {key: np.concatenate([np.asarray(committed[key][nf * L:]).reshape(
                    (-1,) + ins[key].shape[3:]), ins[key][i, r, :j + 1]]) for key in ("k", "v", "beta", "g")}
                check_output(kind, 1.0, go[i:i + 1, r, j], dec, Sg32, Se[None], cp, rc,
                             ins["q"][i:i + 1, r, j], ent["k"][None], ent["v"][None],
                             ent["beta"][None], ent["g"][None], oo[i:i + 1, r, j],
                             "pair %d round %d draft %d" % (i, r, j))
            for key in ins:
                committed[key].extend(list(ins[key][i, r, :int(acc[i, r])]))
