"""Shared helpers of the GPU parity tests: drive the library through the C ABI on seeded inputs,
gather the (sequence, head) pairs under test, and run the fp64 oracle on exactly those inputs.

Tolerance metric for fp32 results (no tolerance is printed on the pages; this is the reading
used throughout): err = |gpu - oracle| / max(|oracle|, rms(oracle over that head's vector or
tile)), required <= 1e-4 elementwise. The rms floor keeps the ratio defined where an output
happens to cancel to ~0.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from oracle import quant
from ssm_decode_state_amd import synth

TOL = 1e-4
RC_FP8_ROW, RC_FP4_B16 = 1, 2  # read-copy kinds (ssm_replay.h)


def rel_err(g: np.ndarray, o: np.ndarray, axes) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    rms = np.sqrt((o ** 2).mean(axis=axes, keepdims=True))
    return np.abs(g - o) / np.maximum(np.maximum(np.abs(o), rms), 1e-30)


def assert_close(g, o, axes, what: str, tol: float = TOL) -> float:
    e = rel_err(g, o, axes)
    worst = float(e.max()) if e.size else 0.0
    if not worst <= tol:
        idx = np.unravel_index(int(np.argmax(e)), e.shape)
        raise AssertionError("%s: max rel err %.3g > %.1g at %s (gpu %r, oracle %r)"
                             % (what, worst, tol, idx, float(np.asarray(g)[idx]),
                                float(np.asarray(o)[idx])))
    return worst


class M2Tokens:
    """Per-step inputs (CPU tensors as drawn) and per-head gathers for the oracle."""

    def __init__(self, shape: synth.Shape, seed: int, tag: str = "decode", layer: int = 0):
        self.shape, self.seed, self.tag, self.layer = shape, seed, tag, layer
        self.steps = []

    def draw(self, index: int, ntok: int = 1):
        d = synth.token_inputs(self.shape, self.seed, self.tag, index, ntok, self.layer)
        self.steps.append(d)
        return d

    def head_inputs(self, pairs):
        """Stack the drawn tokens for each (b, h) pair: x [n][T][P], B/C [n][T][N], dt [n][T]."""
        hpg = self.shape.heads // self.shape.groups
        xs, Bs, Cs, dts = [], [], [], []
        for (b, h) in pairs:
            g = h // hpg
            xs.append(torch.cat([d["x"][b, :, h] for d in self.steps], 0))
            Bs.append(torch.cat([d["B"][b, :, g] for d in self.steps], 0))
            Cs.append(torch.cat([d["C"][b, :, g] for d in self.steps], 0))
            dts.append(torch.cat([d["dt"][b, :, h] for d in self.steps], 0))
        return (synth.to_f64(torch.stack(xs)), synth.to_f64(torch.stack(Bs)),
                synth.to_f64(torch.stack(Cs)), synth.to_f64(torch.stack(dts)))


def sample_pairs(batch: int, heads: int, n: int, seed: int = 123):
    """Corner pairs plus a seeded random sample of (sequence, head) pairs."""
    pairs = {(0, 0), (batch - 1, heads - 1), (0, heads - 1), (batch - 1, 0)}
    rng = np.random.default_rng(seed)
    while len(pairs) < min(n, batch * heads):
        pairs.add((int(rng.integers(batch)), int(rng.integers(heads))))
    return sorted(pairs)


def m2_oracle(A, D, h0, tokens: M2Tokens, pairs, snap_after=()):
    x, B, C, dt = tokens.head_inputs(pairs)
    hs = np.array([h for (_, h) in pairs])
    h0p = None if h0 is None else np.stack([h0[b, h].double().numpy() for (b, h) in pairs])
    return oracle.m2_sequential(A.double().numpy()[hs], D.double().numpy()[hs], h0p, x, B, C, dt,
                                snap_after=snap_after)


def to_dev(d, dev):
    return {k: v.to(dev, non_blocking=True).contiguous() for k, v in d.items()}


class GdnTokens:
    """Per-step GDN inputs and per-head gathers for the oracle."""

    def __init__(self, shape: synth.Shape, seed: int, tag: str = "decode",
                 fast_decay: bool = False):
        self.shape, self.seed, self.tag, self.fast_decay = shape, seed, tag, fast_decay
        self.steps = []

    def draw(self, index: int):
        d = synth.token_inputs(self.shape, self.seed, self.tag, index,
                               fast_decay=self.fast_decay)
        self.steps.append(d)
        return d

    def head_inputs(self, pairs):
        out = []
        for key in ("q", "k", "v", "beta", "g"):
            out.append(synth.to_f64(torch.stack(
                [torch.cat([d[key][b, :, h] for d in self.steps], 0) for (b, h) in pairs])))
        return out


def gdn_oracle(S0, tokens: GdnTokens, pairs, scale=1.0, snap_after=()):
    q, k, v, beta, g = tokens.head_inputs(pairs)
    S0p = None if S0 is None else np.stack([S0[b, h].double().numpy() for (b, h) in pairs])
    return oracle.gdn_sequential(S0p, q, k, v, beta, g, scale=scale, snap_after=snap_after)


# ----------------------------------------------------------------------------------------------
# Read copy: download a state's copy and checkpoint, and check them with the oracle's quantizer
# ----------------------------------------------------------------------------------------------
def copy_of(st, pairs, rc):
    """Codes / scales of the given heads, converted to natural [n][P][N] / [n][P][N/16] order."""
    c, L = st.cfg, st.layout
    B, H, P, N = c.batch, c.heads, c.dim_p, c.dim_n
    idx = torch.tensor([b * H + h for (b, h) in pairs], device=st.mem.device)
    if rc == RC_FP8_ROW:
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


def ckpt_of(st, pairs):
    """The GPU's fp32 checkpoint tiles of the given heads, natural [n][P][N] (exact fp32 bits)."""
    c = st.cfg
    P, N = c.dim_p, c.dim_n
    nat = st.region(st.layout.off_ckpt, c.batch * c.heads * P * N * 4).view(torch.float32)
    nat = nat.view(c.batch * c.heads, N // 4, P, 4)
    idx = torch.tensor([b * c.heads + h for (b, h) in pairs], device=st.mem.device)
    return nat.index_select(0, idx).permute(0, 2, 1, 3).reshape(len(pairs), P, N).cpu().numpy()


def quantize(h, rc):
    return quant.fp8_row_quantize(h) if rc == RC_FP8_ROW else quant.fp4_quantize(h)


def decode_copy(copy, rc):
    return (quant.fp8_row_decode(*copy) if rc == RC_FP8_ROW
            else quant.fp4_decode(*copy)).astype(np.float64)


def elem_bound(h32, copy, rc):
    """Closed-form element bound of the copy around the fp32 tile h32, with the copy's scales."""
    if rc == RC_FP8_ROW:
        return quant.fp8_row_bound(h32, copy[1])
    return quant.fp4_bound(h32, quant.fp4_scales(copy[1], copy[2]))


def assert_copy_exact(h32, copy, rc, what):
    exp = quantize(h32, rc)
    for i, (g, e) in enumerate(zip(copy, exp)):
        np.testing.assert_array_equal(np.asarray(g), np.asarray(e), err_msg="%s (part %d)" % (what, i))


def drift_slope(per_window):
    """Least-squares slope of per-window values and its standard error."""
    y = np.asarray(per_window, dtype=np.float64)
    t = np.arange(len(y), dtype=np.float64)
    tc = t - t.mean()
    slope = float((tc * (y - y.mean())).sum() / (tc ** 2).sum())
    res = y - y.mean() - slope * tc
    se = float(np.sqrt((res ** 2).sum() / max(len(y) - 2, 1) / (tc ** 2).sum()))
    return slope, se


def report_drift(rec):
    print("read-copy drift:", json.dumps(rec))
    out = os.environ.get("SSM_DRIFT_OUT")
    if out:
        with open(out, "a") as f:
            f.write(json.dumps(rec) + "\n")


def adversarial_tiles(P, N, seed):
    """P x N fp32 tiles that stress the copy's scales: random; one huge element with everything
    else deep in the subnormal range of the format; a block whose scale underflows next to a large
    element; all zero; Cauchy tails; rows far below 448 * 2^-126 (scale floor) beside zero rows;
    one row of exact midpoints at scale 1 and a row at the floor boundary."""
    rng = np.random.default_rng(seed)
    tiles = [rng.standard_normal((P, N)).astype(np.float32) * 0.3]
    t = (rng.standard_normal((P, N)) * 1e-3).astype(np.float32)
    t[3, 5] = 50.0
    tiles.append(t)
    t = np.zeros((P, N), np.float32)
    t[0, :16] = 1e-30
    t[5, 7] = 2.0
    t[9, 16:32] = rng.standard_normal(16).astype(np.float32) * 1e-12
    tiles.append(t)
    tiles.append(np.zeros((P, N), np.float32))
    tiles.append((rng.standard_cauchy((P, N)) * 0.1).astype(np.float32))
    t = np.zeros((P, N), np.float32)
    t[::2] = (rng.choice([-1.0, 1.0], (P // 2, N)) * rng.uniform(1.2e-38, 2e-37, (P // 2, N)))
    t[1, :] = 0.0
    tiles.append(t.astype(np.float32))
    t = (rng.standard_normal((P, N)) * 0.2).astype(np.float32)
    mids = [448.0] + [2.0 ** e * (1 + 1 / 16) for e in range(-6, 8)] + [2.0 ** -10, 3 * 2.0 ** -10]
    t[0] = 0.0
    t[0, :len(mids)] = mids
    t[1] = 0.0
    t[1, 0] = np.float32(448 * 2.0 ** -126)
    tiles.append(t)
    return tiles
