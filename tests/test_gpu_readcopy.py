"""GPU checks of the low-precision read copy (Mamba-2, P = 64).

The copy is written from the fp32 checkpoint at init and at every flush and read only by the
output path; the recurrence never sees it (news article, para 4). Checks, in every window:
  * copy: the codes and scales the GPU wrote equal, bit for bit, the oracle's fp32 quantizer
    applied to the GPU's own fp32 checkpoint (at init: to the initial state);
  * outputs: every replayed output equals, to 1e-4 (the fp32 metric of harness.py), the oracle's
    replay form evaluated on the GPU's decoded copy -- the copy is the only thing that differs
    from the exact output; the window-closing step folds in fp32 and emits its output from the new
    fp32 checkpoint, so it is compared with the exact output at 1e-4;
  * bound: every replayed output is within
        |y - y_exact| <= e^{s0} sum_n |C[n]| (bound[p, n] + |h_gpu - h_exact|[p, n]) + 1e-4 m
    of the exact fp64 output, with bound the closed-form element bound of the format evaluated on
    the GPU's fp32 checkpoint with its own scales (oracle.quant), the second term the fp32
    checkpoint's own deviation from the fp64 one, and m = max(|y_copy|, rms) the 1e-4 metric's
    floor for the fp32 arithmetic of the replay;
  * fp32 recurrence: every flushed checkpoint matches the oracle to 1e-4;
  * no drift: the least-squares slope of the per-window worst err / bound over the windows is not
    positive beyond three standard errors (the rounding never enters the recurrence, so later
    windows are no worse than earlier ones). The slopes are printed and, when the environment
    names a file in SSM_DRIFT_OUT, appended to it as JSON lines.
Adversarial tiles (zero rows and tiles, a block whose scale underflows, one huge element, Cauchy
tails, rows far below 448 * 2^-126 that need the scale floor, exact midpoints) go through the same
copy and output checks.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import (M2Tokens, TOL, assert_close, assert_copy_exact, ckpt_of, copy_of, decode_copy,
                     drift_slope, elem_bound, m2_oracle, report_drift, sample_pairs, to_dev,
                     adversarial_tiles)
from oracle import quant
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def make(shape, seed, rc, h0=None):
    A, D = synth.head_constants(shape, seed)
    if h0 is None:
        h0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(bd.SSM_MAMBA2, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, shape.window, 1,
                         bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc)
    st = bd.State(cfg, h0.to(DEV), A.to(DEV), D.to(DEV))
    return st, A, D, h0


@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("B,H,N", [(2, 4, 64), (3, 5, 128)])
def test_init_copy_is_bit_exact(rc, B, H, N):
    shape = synth.Shape(synth.MAMBA2, B, H, H, 64, N, 8, 1)
    st, A, D, h0 = make(shape, 50 + N, rc)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    torch.cuda.synchronize()
    assert_copy_exact(np.stack([h0[b, h].numpy() for (b, h) in pairs]), copy_of(st, pairs, rc), rc,
                      "init copy")


def run_readcopy(shape, seed, rc, T, pairs, h0=None):
    """Decode T lock-step tokens; check copies, outputs, bounds and checkpoints window by window.
    Returns the per-window worst err / bound."""
    L = shape.window
    st, A, D, h0 = make(shape, seed, rc, h0)
    tok = M2Tokens(shape, seed)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    y = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    torch.cuda.synchronize()
    cks, copies = [ckpt_of(st, pairs)], [copy_of(st, pairs, rc)]  # each window's start
    ys = []
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), y)
        ys.append(y[bi, hi].clone())
        if (t + 1) % L == 0:
            cks.append(ckpt_of(st, pairs))
            copies.append(copy_of(st, pairs, rc))
    torch.cuda.synchronize()
    gy = torch.stack(ys, 1).cpu().double().numpy()
    nwin = T // L
    oy, _, osn = m2_oracle(A, D, h0, tok, pairs, snap_after=list(range(L, T + 1, L)))
    x, Bm, Cm, dt = tok.head_inputs(pairs)
    hs = np.array([h for (_, h) in pairs])
    Ah, Dh = A.double().numpy()[hs], D.double().numpy()[hs]
    h0n = np.stack([h0[b, h].double().numpy() for (b, h) in pairs])
    # fp32 recurrence untouched by the copy
    if nwin:
        assert_close(np.stack(cks[1:nwin + 1], 1), osn, (-2, -1), "flushed fp32 checkpoints")
    for w, (hg32, cp) in enumerate(zip(cks, copies)):  # init and every flush
        assert_copy_exact(hg32, cp, rc, "copy written at the start of window %d" % w)
    per_window = []
    for w in range((T + L - 1) // L):
        hg32, cp = cks[w], copies[w]
        he = h0n if w == 0 else osn[:, w - 1]
        dec = decode_copy(cp, rc)
        lim_el = elem_bound(hg32, cp, rc) + np.abs(hg32.astype(np.float64) - he)
        worst = 0.0
        for k in range(1, L + 1):
            t = w * L + k - 1
            if t >= T:
                break
            if k == L:  # the fused window-closing step: output from the new fp32 checkpoint
                assert_close(gy[:, t], oy[:, t], (-1,), "window-closing output (t=%d)" % t)
                continue
            e = slice(w * L, t + 1)  # the window's entries through this token
            yc = np.stack([oracle.m2_replay_output(float(Ah[i]), float(Dh[i]), dec[i], x[i, e],
                                                   Bm[i, e], Cm[i, t], dt[i, e])
                           for i in range(len(pairs))])
            assert_close(gy[:, t], yc, (-1,), "outputs on the decoded copy (window %d, k=%d)" % (w, k))
            s0 = np.exp(Ah * dt[:, e].sum(axis=1))
            lim = quant.output_bound(lim_el, Cm[:, t], s0)
            rms = np.sqrt((yc ** 2).mean(axis=-1, keepdims=True))
            slack = TOL * np.maximum(np.abs(yc), rms)
            err = np.abs(gy[:, t] - oy[:, t])
            assert np.all(err <= lim + slack), (w, k, float((err - lim - slack).max()))
            worst = max(worst, float((err / (lim + slack)).max()))
        per_window.append(worst)
    return per_window


@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("case", ["small", "small_f32", "serving"])
def test_readcopy_decode(rc, case):
    if case.startswith("small"):  # small_f32: fp32 inputs
        shape = synth.Shape(synth.MAMBA2, 2, 6, 3, 64, 128, 8, 1, in_bf16=case == "small")
        seed, T = 60 + rc + (3 if case == "small_f32" else 0), 96
        pairs = [(b, h) for b in range(2) for h in range(6)]
    else:
        w = synth.WORKLOADS["m2_b256_readcopy"]
        shape, seed, T = w["shape"], w["seed"], w["steps"]
        pairs = sample_pairs(shape.batch, shape.heads, 12)
    per_window = run_readcopy(shape, seed, rc, T, pairs)
    slope, se = drift_slope(per_window)
    report_drift({"layer": "mamba2", "case": case, "format": "fp8" if rc == 1 else "fp4",
                  "windows": len(per_window), "slope_per_window": slope, "stderr": se,
                  "mean_err_over_bound": float(np.mean(per_window)),
                  "max_err_over_bound": float(np.max(per_window))})
    assert slope <= 3 * se + 1e-9, (slope, se, per_window)


@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("N", [64, 128])
def test_adversarial_tiles(rc, N):
    """The copy of adversarial initial states is bit-exact on the GPU, every replayed output
    matches the oracle on the decoded copy and stays within the bound, and after the first fold
    the rewritten copy is bit-exact again."""
    tiles = adversarial_tiles(64, N, 70 + N + rc)
    H = len(tiles)
    shape = synth.Shape(synth.MAMBA2, 2, H, H, 64, N, 8, 1)
    h0 = torch.from_numpy(np.stack([np.stack(tiles), np.stack(tiles[::-1])]))
    pairs = [(b, h) for b in range(2) for h in range(H)]
    per_window = run_readcopy(shape, 75 + N + rc, rc, 12, pairs, h0=h0)
    assert len(per_window) == 2


@pytest.mark.parametrize("rc", [1, 2])
def test_readcopy_speculative_rounds(rc):
    """Drafts verified through the read copy (several queries per call). After every round
    (rollback and any fold) the copy is bit-exact against the GPU's own fp32 checkpoint; every
    draft output equals, to 1e-4, the oracle's replay form on the decoded copy in effect for that
    round, over the committed entries since the last fold and drafts 1..j, and lies within the
    bound around the exact speculative output; the fp32 checkpoint after the rounds is exact."""
    shape = synth.Shape(synth.MAMBA2, 2, 6, 3, 64, 128, 8, 4)
    seed, R, S = 70 + rc, 12, shape.max_draft
    L, hpg = shape.window, shape.heads // shape.groups
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(bd.SSM_MAMBA2, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, L, S, bd.SSM_IN_BF16, rc)
    st = bd.State(cfg, h0.to(DEV), A.to(DEV), D.to(DEV))
    pairs = [(b, h) for b in range(shape.batch) for h in range(shape.heads)]
    n = len(pairs)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    y = torch.empty(shape.batch, S, shape.heads, shape.dim_p, device=DEV)
    torch.cuda.synchronize()
    cks, copies = [ckpt_of(st, pairs)], [copy_of(st, pairs, rc)]  # in effect for round r: index r
    outs, drafts, accs = [], [], []
    for r in range(R):
        d = synth.token_inputs(shape, seed, "draft", r, ntok=S)
        drafts.append(d)
        bd.ssm_spec_append(st, S, to_dev(d, DEV), y)
        outs.append(y[bi, :, hi].clone())
        acc = synth.accept_counts(shape.batch, S, 1003, r)
        accs.append(acc)
        bd.ssm_spec_rollback(st, acc.to(DEV))
        cks.append(ckpt_of(st, pairs))
        copies.append(copy_of(st, pairs, rc))
    torch.cuda.synchronize()
    for r, (hg32, cp) in enumerate(zip(cks, copies)):
        assert_copy_exact(hg32, cp, rc, "copy after round %d" % (r - 1))
    gy = torch.stack(outs, 1).cpu().double().numpy()  # [n][R][S][P]
    x = np.stack([np.stack([synth.to_f64(d["x"][b, :, h]) for d in drafts]) for (b, h) in pairs])
    Bm = np.stack([np.stack([synth.to_f64(d["B"][b, :, h // hpg]) for d in drafts]) for (b, h) in pairs])
    Cm = np.stack([np.stack([synth.to_f64(d["C"][b, :, h // hpg]) for d in drafts]) for (b, h) in pairs])
    dt = np.stack([np.stack([synth.to_f64(d["dt"][b, :, h]) for d in drafts]) for (b, h) in pairs])
    acc = np.stack([torch.stack(accs, 1)[b].numpy() for (b, _) in pairs]).astype(np.int32)
    hs = np.array([h for (_, h) in pairs])
    Ah, Dh = A.double().numpy()[hs], D.double().numpy()[hs]
    h0n = np.stack([h0[b, h].double().numpy() for (b, h) in pairs])
    tot = np.cumsum(acc, axis=1)
    folds = [list(range(L, int(tot[i, -1]) + 1, L)) for i in range(n)]
    snap = np.full((n, max(1, max(len(f) for f in folds))), -1, dtype=np.int32)
    for i, f in enumerate(folds):
        snap[i, :len(f)] = f
    oy, _, sn = oracle.m2_spec_rounds(Ah, Dh, h0n, x, Bm, Cm, dt, acc, snap_after=snap)
    assert max(len(f) for f in folds) >= 2  # the rounds cross several folds
    for i in range(n):
        com = {"x": [], "B": [], "dt": []}  # the accepted drafts, in order
        for r in range(R):
            nf = len(com["dt"]) // L  # folds so far
            he = h0n[i] if nf == 0 else sn[i, nf - 1]
            hg32, cp = cks[r][i:i + 1], tuple(c[i:i + 1] for c in copies[r])
            dec = decode_copy(cp, rc)[0]
            lim_el = (elem_bound(hg32, cp, rc) + np.abs(hg32.astype(np.float64) - he))[0]
            for j in range(S):
                ent = {"x": np.concatenate([np.asarray(com["x"][nf * L:]).reshape(-1, shape.dim_p), x[i, r, :j + 1]]),
                       "B": np.concatenate([np.asarray(com["B"][nf * L:]).reshape(-1, shape.dim_n), Bm[i, r, :j + 1]]),
                       "dt": np.concatenate([np.asarray(com["dt"][nf * L:]).reshape(-1), dt[i, r, :j + 1]])}
                yc = oracle.m2_replay_output(float(Ah[i]), float(Dh[i]), dec, ent["x"], ent["B"],
                                             Cm[i, r, j], ent["dt"])
                what = "pair %d round %d draft %d" % (i, r, j)
                assert_close(gy[i, r, j], yc, (-1,), "output on the decoded copy, " + what)
                s0 = np.exp(Ah[i] * ent["dt"].sum())
                lim = quant.output_bound(lim_el, Cm[i, r, j], s0)
                rms = np.sqrt((yc ** 2).mean())
                slack = TOL * np.maximum(np.abs(yc), rms)
                err = np.abs(gy[i, r, j] - oy[i, r, j])
                assert np.all(err <= lim + slack), (what, float((err - lim - slack).max()))
            for key, src in (("x", x), ("B", Bm), ("dt", dt)):
                com[key].extend(list(src[i, r, :int(acc[i, r])]))
    nat = torch.empty(shape.batch, shape.heads, shape.dim_p, shape.dim_n, device=DEV)
    bd.ssm_flush(st, bd.SSM_FLUSH_ALL)
    bd.ssm_ckpt_export(st, nat)
    torch.cuda.synchronize()
    _, hT, _ = oracle.m2_spec_rounds(Ah, Dh, h0n, x, Bm, Cm, dt, acc)
    got = np.stack([nat[b, h].cpu().double().numpy() for (b, h) in pairs])
    assert_close(got, hT, (-2, -1), "fp32 checkpoint after the speculative rounds")
