"""Shared helpers of the GPU parity tests: drive the library through the C ABI on seeded inputs,
gather the (sequence, head) pairs under test, and run the fp64 oracle on exactly those inputs.

Tolerance metric for fp32 results (no tolerance is printed on the pages; this is the reading
used throughout): err = |gpu - oracle| / max(|oracle|, rms(oracle over that head's vector or
tile)), required <= 1e-4 elementwise. The rms floor keeps the ratio defined where an output
happens to cancel to ~0.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from ssm_decode_state_amd import synth

TOL = 1e-4


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

    def __init__(self, shape: synth.Shape, seed: int, tag: str = "decode"):
        self.shape, self.seed, self.tag = shape, seed, tag
        self.steps = []

    def draw(self, index: int):
        d = synth.token_inputs(self.shape, self.seed, self.tag, index)
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
