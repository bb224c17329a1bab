"""GPU checks of the low-precision read copy (Mamba-2, P = 64).

The copy is written from the fp32 checkpoint at init and at every flush and read only by the
output path; the recurrence never sees it. Checks:
  * at init the copy's codes and scales equal, bit for bit, the oracle's fp32 emulation of the
    quantizer applied to the same initial checkpoint;
  * every output stays within the closed-form bound of the quantization error around the exact
    (fp64, unquantized) output;
  * every flushed fp32 checkpoint still matches the oracle to 1e-4 (no feedback of rounded values);
  * no drift: the worst error/bound ratio does not grow from window to window;
  * after each flush the copy equals the oracle's quantization of its own fp64 checkpoint except
    for codes within a rounding step (counted and bounded).
"""
import numpy as np
import pytest
import torch

from harness import M2Tokens, assert_close, m2_oracle, sample_pairs, to_dev
from oracle import quant
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")


def copy_of(st, pairs, rc):
    """Codes / scales of the given heads, converted to natural [n][P][N] / [n][P][N/16] order."""
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


def make(shape, seed, rc):
    A, D = synth.head_constants(shape, seed)
    h0 = synth.initial_state(shape, seed, 0.3162)
    cfg = bd.make_config(bd.SSM_MAMBA2, shape.batch, shape.heads, shape.groups, shape.dim_p,
                         shape.dim_n, shape.window, 1, bd.SSM_IN_BF16, rc)
    st = bd.State(cfg, h0.to(DEV), A.to(DEV), D.to(DEV))
    return st, A, D, h0


def emulate(h, rc):
    if rc == bd.SSM_RC_FP8_ROW:
        return quant.fp8_row_quantize(h)
    return quant.fp4_quantize(h)


def decoded_and_bound(h64, rc):
    """Oracle quantization of an fp64 checkpoint (cast to fp32): decoded copy and error bound."""
    h = h64.astype(np.float32)
    if rc == bd.SSM_RC_FP8_ROW:
        c, s = quant.fp8_row_quantize(h)
        return quant.fp8_row_decode(c, s), quant.fp8_row_bound(h, s)
    c, sb, st = quant.fp4_quantize(h)
    return quant.fp4_decode(c, sb, st), quant.fp4_bound(h, quant.fp4_scales(sb, st))


@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("B,H,N", [(2, 4, 64), (3, 5, 128)])
def test_init_copy_is_bit_exact(rc, B, H, N):
    shape = synth.Shape(synth.MAMBA2, B, H, H, 64, N, 8, 1)
    st, A, D, h0 = make(shape, 50 + N, rc)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    torch.cuda.synchronize()
    got = copy_of(st, pairs, rc)
    exp = emulate(np.stack([h0[b, h].numpy() for (b, h) in pairs]), rc)
    for g, e in zip(got, exp):
        np.testing.assert_array_equal(np.asarray(g), np.asarray(e))


@pytest.mark.parametrize("rc", [1, 2])
@pytest.mark.parametrize("case", ["small", "serving"])
def test_readcopy_decode(rc, case):
    if case == "small":
        shape = synth.Shape(synth.MAMBA2, 2, 6, 3, 64, 128, 8, 1)
        seed, T = 60 + rc, 96
        pairs = [(b, h) for b in range(2) for h in range(6)]
    else:
        w = synth.WORKLOADS["m2_b256_readcopy"]
        shape, seed, T = w["shape"], w["seed"], w["steps"]
        pairs = sample_pairs(shape.batch, shape.heads, 12)
    L = shape.window
    st, A, D, h0 = make(shape, seed, rc)
    tok = M2Tokens(shape, seed)
    bi = torch.tensor([b for (b, _) in pairs], device=DEV)
    hi = torch.tensor([h for (_, h) in pairs], device=DEV)
    y = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)
    ys, cks, copies = [], [], []
    P, N = shape.dim_p, shape.dim_n
    for t in range(T):
        bd.ssm_replay_decode(st, to_dev(tok.draw(t), DEV), y)
        ys.append(y[bi, hi].clone())
        if (t + 1) % L == 0:
            nat = st.region(st.layout.off_ckpt, shape.batch * shape.heads * P * N * 4)
            nat = nat.view(torch.float32).view(shape.batch * shape.heads, N // 4, P, 4)
            idx = torch.tensor([b * shape.heads + h for (b, h) in pairs], device=DEV)
            cks.append(nat.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N)
                       .cpu().double().numpy())
            copies.append(copy_of(st, pairs, rc))
    torch.cuda.synchronize()
    gy = torch.stack(ys, 1).cpu().double().numpy()
    snaps = list(range(L, T + 1, L))
    oy, _, osn = m2_oracle(A, D, h0, tok, pairs, snap_after=snaps)
    # (a) the fp32 recurrence is untouched by the copy
    assert_close(np.stack(cks, 1), osn, (-2, -1), "flushed fp32 checkpoints")
    # (b) every output within the bound around the exact output
    x, Bm, Cm, dt = tok.head_inputs(pairs)
    hs = np.array([h for (_, h) in pairs])
    Ah = A.double().numpy()[hs]
    ratios = []
    h0n = np.stack([h0[b, h].double().numpy() for (b, h) in pairs])
    for wdw in range(T // L):
        hc = h0n if wdw == 0 else osn[:, wdw - 1]
        _, bnd = decoded_and_bound(hc, rc)
        for k in range(1, L + 1):
            t = wdw * L + k - 1
            s0 = np.exp(Ah * dt[:, wdw * L:t + 1].sum(axis=1))
            lim = s0[:, None] * np.einsum("ipn,in->ip", bnd, np.abs(Cm[:, t]))
            yo = oy[:, t]
            rms = np.sqrt((yo ** 2).mean(axis=-1, keepdims=True))
            slack = 2e-4 * np.maximum(np.abs(yo), rms)
            err = np.abs(gy[:, t] - yo)
            assert np.all(err <= lim * 1.001 + slack), (wdw, k, float((err - lim).max()))
            ratios.append(float((err / (lim + slack)).max()))
    per_window = np.array(ratios).reshape(T // L, L).max(axis=1)
    # (c) no drift: later windows are no worse than the first ones beyond noise
    half = len(per_window) // 2
    assert per_window[half:].max() <= 1.5 * per_window[:half].max() + 0.05, per_window
    # (d) the copy written at each flush is the quantization of the flushed checkpoint
    for wdw, cp in enumerate(copies):
        exp = emulate(osn[:, wdw].astype(np.float32), rc)
        gc, ec = np.asarray(cp[0]), np.asarray(exp[0])
        mism = gc != ec
        assert mism.mean() < 0.01, mism.mean()
        if rc == bd.SSM_RC_FP8_ROW:  # row scales agree to an ulp: codes differ by one step at most
            mag_g, mag_e = (gc & 0x7F).astype(int), (ec & 0x7F).astype(int)
            assert np.all(np.abs(mag_g - mag_e)[mism] <= 1)
        else:  # block scales may step at a tie, which moves a whole block: count those too
            assert (np.asarray(cp[1]) != np.asarray(exp[1])).mean() < 0.01
