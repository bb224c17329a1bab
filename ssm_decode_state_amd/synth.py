"""Seeded synthetic inputs for the ReplaySSM decode workloads.

This module holds the input distributions only, none of the method's arithmetic. The oracle-side
tests and the HIP path both consume the exact bits produced here (bf16/fp32 values are rounded
once, here, and the oracle upcasts those bits to fp64).

Distributions (Mamba-2 workloads):
  x ~ N(0, 1); B, C ~ N(0, 1/N); dt = softplus(z), z ~ N(-2, 0.5) (second parameter = variance);
  A = -exp(U(0, 2)) and D ~ N(0, 1), one scalar per head; checkpoint h0 ~ N(0, 0.1) or zero.
Distributions (Gated DeltaNet workloads):
  q, k ~ N(0, I) then L2-normalised in fp64 before rounding; v ~ N(0, 1);
  beta = sigmoid(N(0, 1)); g = -softplus(N(0, 1)) (a log-decay); S0 ~ N(0, 0.1) or zero.

Every draw goes through torch's CPU generator (mt19937) seeded from a 63-bit hash of
(seed, stream tag, index), so any (tag, index) block can be regenerated on its own. Draws are made
in fp32 (normals) or fp64 (the values that pass through softplus/sigmoid/exp/normalisation), then
rounded to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import torch

MAMBA2 = 0
GDN = 1
KDA = 2


@dataclasses.dataclass(frozen=True)
class Shape:
    """Problem shape of one SSM layer (names follow the pages' two layer types)."""
    kind: int          # MAMBA2, GDN or KDA
    batch: int         # sequences
    heads: int         # H
    groups: int        # Mamba-2: B/C groups G (H % G == 0); GDN: == heads
    dim_p: int         # Mamba-2 head dim P; GDN value dim dv (rows of the state tile)
    dim_n: int         # Mamba-2 state dim N; GDN key dim dk (columns of the state tile)
    window: int        # flush window L
    max_draft: int = 1  # largest speculative draft count per append
    in_bf16: bool = True  # x/B/C (q/k/v) storage dtype: bf16 if True, else fp32

    @property
    def in_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.in_bf16 else torch.float32


# A small parity case and the serving-batch cases.
WORKLOADS: Dict[str, dict] = {
    "m2_small": dict(shape=Shape(MAMBA2, 2, 4, 4, 16, 16, 4, 4, in_bf16=False), steps=64, seed=0,
                     h0_std=0.0),
    "m2_b256": dict(shape=Shape(MAMBA2, 256, 128, 128, 64, 128, 16, 1), steps=256, seed=1,
                    h0_std=math.sqrt(0.1)),
    "m2_b256_spec": dict(shape=Shape(MAMBA2, 256, 128, 128, 64, 128, 16, 4), rounds=128, ndraft=4,
                         seed=2, accept_seed=1002, h0_std=math.sqrt(0.1)),
    "m2_b256_readcopy": dict(shape=Shape(MAMBA2, 256, 128, 128, 64, 128, 16, 1), steps=512, seed=3,
                             h0_std=math.sqrt(0.1)),
    "gdn_b256": dict(shape=Shape(GDN, 256, 32, 32, 128, 128, 16, 1), steps=256, seed=4,
                     h0_std=math.sqrt(0.1)),
    "gdn_b256_spec": dict(shape=Shape(GDN, 256, 32, 32, 128, 128, 16, 4), rounds=128, ndraft=4,
                          seed=5, accept_seed=1002, h0_std=math.sqrt(0.1)),
    "kda_b256": dict(shape=Shape(KDA, 256, 32, 32, 128, 128, 16, 1), steps=256, seed=6,
                     h0_std=math.sqrt(0.1)),
}


def derive_seed(*parts) -> int:
    """63-bit seed from a tuple of ints/strings (blake2b of their repr)."""
    h = hashlib.blake2b(repr(tuple(parts)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(*parts) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(derive_seed(*parts))


def _softplus64(z: torch.Tensor) -> torch.Tensor:
    # log(1 + e^z) evaluated stably in fp64
    return torch.where(z > 20, z, torch.log1p(torch.exp(torch.clamp(z, max=20.0))))


def head_constants(shape: Shape, seed: int, layer: int = 0):
    """Mamba-2 per-head A < 0 and D (fp32, [H]). GDN layers have none (returns None, None)."""
    if shape.kind != MAMBA2:
        return None, None
    g = _gen(seed, "const", layer)
    u = torch.rand(shape.heads, generator=g, dtype=torch.float64) * 2.0
    A = (-torch.exp(u)).to(torch.float32)
    D = torch.randn(shape.heads, generator=g, dtype=torch.float32)
    return A, D


def initial_state(shape: Shape, seed: int, std: float, layer: int = 0,
                  batch_slice: Optional[slice] = None) -> torch.Tensor:
    """Prefilled checkpoint, fp32, natural layout [batch][H][P][N] (N fastest).

    Drawn per sequence, so a slice of sequences can be regenerated alone."""
    bs = range(shape.batch)[batch_slice] if batch_slice is not None else range(shape.batch)
    out = torch.zeros(len(bs), shape.heads, shape.dim_p, shape.dim_n, dtype=torch.float32)
    if std == 0.0:
        return out
    s = torch.tensor(std, dtype=torch.float32)
    for i, b in enumerate(bs):
        g = _gen(seed, "h0", layer, b)
        out[i] = torch.randn(shape.heads, shape.dim_p, shape.dim_n, generator=g) * s
    return out


def token_inputs(shape: Shape, seed: int, tag: str, index: int, ntok: int = 1,
                 layer: int = 0, fast_decay: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of `ntok` consecutive tokens for every sequence, as one block keyed by (tag, index).

    Mamba-2: x [batch][ntok][H][P], B and C [batch][ntok][G][N] in the storage dtype;
             dt [batch][ntok][H] fp32.
    GDN:     q, k [batch][ntok][H][dk], v [batch][ntok][H][dv] in the storage dtype;
             beta, g [batch][ntok][H] fp32.
    KDA:     as GDN with g [batch][ntok][H][dk] (one log-decay per key channel).
    fast_decay (GDN, KDA): a third of the decays are redrawn as g = -U(10, 40) per token -- the
    key channels n % 3 == 0 (KDA) or the heads h % 3 == 0 (GDN) -- from a stream of their own,
    so every other value is unchanged: gates that forget a channel within a token or two.
    """
    g = _gen(seed, tag, layer, index)
    bsz, H = shape.batch, shape.heads
    dt_ = shape.in_dtype
    if shape.kind == MAMBA2:
        G, P, N = shape.groups, shape.dim_p, shape.dim_n
        sN = torch.tensor(math.sqrt(1.0 / N), dtype=torch.float32)
        x = torch.randn(bsz, ntok, H, P, generator=g).to(dt_)
        Bm = (torch.randn(bsz, ntok, G, N, generator=g) * sN).to(dt_)
        Cm = (torch.randn(bsz, ntok, G, N, generator=g) * sN).to(dt_)
        z = torch.randn(bsz, ntok, H, generator=g, dtype=torch.float64) * math.sqrt(0.5) - 2.0
        dt = _softplus64(z).to(torch.float32)
        return {"x": x, "B": Bm, "C": Cm, "dt": dt}
    dv, dk = shape.dim_p, shape.dim_n
    q = torch.randn(bsz, ntok, H, dk, generator=g, dtype=torch.float64)
    k = torch.randn(bsz, ntok, H, dk, generator=g, dtype=torch.float64)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(bsz, ntok, H, dv, generator=g)
    beta = torch.sigmoid(torch.randn(bsz, ntok, H, generator=g, dtype=torch.float64))
    gshape = (bsz, ntok, H, dk) if shape.kind == KDA else (bsz, ntok, H)
    gl = -_softplus64(torch.randn(*gshape, generator=g, dtype=torch.float64))
    if fast_decay:
        fast = -(10.0 + 30.0 * torch.rand(*gshape, generator=_gen(seed, tag, layer, index, "fast"),
                                          dtype=torch.float64))
        sel = torch.zeros(gshape[-1], dtype=torch.bool)
        sel[::3] = True
        gl = torch.where(sel, fast, gl)
    return {"q": q.to(torch.float32).to(dt_), "k": k.to(torch.float32).to(dt_), "v": v.to(dt_),
            "beta": beta.to(torch.float32), "g": gl.to(torch.float32)}


def token_inputs_device(shape: Shape, seed: int, tag: str, index: int, ntok: int = 1,
                        layer: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    """Same distributions as token_inputs, drawn on the device with a seeded device generator
    (used where only throughput matters and hundreds of steps of inputs must be resident in HBM
    quickly; the values differ from the host stream, so parity tests use token_inputs)."""
    g = torch.Generator(device=device).manual_seed(derive_seed(seed, tag, layer, index, "dev"))
    bsz, H = shape.batch, shape.heads
    dt_ = shape.in_dtype
    kw = dict(generator=g, device=device)
    if shape.kind == MAMBA2:
        G, P, N = shape.groups, shape.dim_p, shape.dim_n
        sN = math.sqrt(1.0 / N)
        x = torch.randn(bsz, ntok, H, P, **kw).to(dt_)
        Bm = (torch.randn(bsz, ntok, G, N, **kw) * sN).to(dt_)
        Cm = (torch.randn(bsz, ntok, G, N, **kw) * sN).to(dt_)
        z = torch.randn(bsz, ntok, H, dtype=torch.float64, **kw) * math.sqrt(0.5) - 2.0
        return {"x": x, "B": Bm, "C": Cm, "dt": _softplus64(z).to(torch.float32)}
    dv, dk = shape.dim_p, shape.dim_n
    q = torch.randn(bsz, ntok, H, dk, dtype=torch.float64, **kw)
    k = torch.randn(bsz, ntok, H, dk, dtype=torch.float64, **kw)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(bsz, ntok, H, dv, **kw)
    beta = torch.sigmoid(torch.randn(bsz, ntok, H, dtype=torch.float64, **kw))
    gshape = (bsz, ntok, H, dk) if shape.kind == KDA else (bsz, ntok, H)
    gl = -_softplus64(torch.randn(*gshape, dtype=torch.float64, **kw))
    return {"q": q.to(torch.float32).to(dt_), "k": k.to(torch.float32).to(dt_), "v": v.to(dt_),
            "beta": beta.to(torch.float32), "g": gl.to(torch.float32)}


def initial_state_device(shape: Shape, seed: int, std: float, layer: int = 0,
                         device="cuda") -> torch.Tensor:
    """Prefilled checkpoint drawn on the device (same distribution as initial_state)."""
    g = torch.Generator(device=device).manual_seed(derive_seed(seed, "h0dev", layer))
    out = torch.randn(shape.batch, shape.heads, shape.dim_p, shape.dim_n, generator=g,
                      device=device)
    return out.mul_(std)


def accept_counts(batch: int, ndraft: int, seed: int, round_index: int) -> torch.Tensor:
    """Per-sequence accepted draft counts, uniform over {0, ..., ndraft}, int32 [batch]."""
    g = _gen(seed, "accept", round_index)
    return torch.randint(0, ndraft + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)


def to_f64(t: torch.Tensor):
    """Exact upcast of stored input bits to a float64 numpy array (for the fp64 oracle)."""
    return t.to(torch.float64).numpy()
