"""Read-copy quantizer emulation (fp32 numpy) and error bounds -- TEST INFRASTRUCTURE ONLY.

The news article (deskofai.com, "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model
Decoding", para 4) describes a high-precision checkpoint that carries the recurrence next to a
low-precision copy used only for reads, evaluated with NVFP4 reads. The pages fix no recipe; the
reading implemented here (and by the HIP read-copy writer) is:

fp8 row copy (OCP FP8 E4M3: bias 7, max 448, no infinity, 0x7F/0xFF NaN), one fp32 scale per row:
    amax = max_n |h[p, n]|;  s = max(amax / 448, 2^-126) (fp32 division) or 1 if amax == 0
    inv = 1 / s;  code = RNE_sat_e4m3(h * inv);  Q(h) = value(code) * s
fp4 block copy (OCP E2M1 values {0, .5, 1, 1.5, 2, 3, 4, 6}), NVFP4-style two-level scale:
    s_t = max(amax_tile / 2688, 2^-117) (2688 = 6 * 448) or 1 if the tile is all zero (fp32, one
    per head tile); per 16 consecutive elements of a row: s_b = value(RNE_sat_e4m3(amax_blk /
    (6 * s_t))), S = s_b * s_t;  code = RNE_sat_e2m1(h * (1 / S)), or 0 for the whole block when
    S == 0;  Q(h) = value(code) * S
The floors keep every scale a normal fp32 number whose reciprocal is finite: 2^-126 is the
smallest normal fp32, and with s_t >= 2^-117 every nonzero block scale (>= 2^-9, the smallest
E4M3 subnormal) gives S >= 2^-126. Without them a row or tile whose largest magnitude is below
about 448 (2688) times 2^-126 gets a subnormal scale, an infinite reciprocal, and 0 * inf = NaN
codes. Above those magnitudes the floors change nothing.
Every arithmetic step is one IEEE fp32 operation (numpy float32 is correctly rounded), so the
codes are a pure function of the fp32 input tile.

Error bounds: round-to-nearest onto a floating-point grid errs by at most half the grid spacing
of the binade holding the scaled value v = |h| / scale (the subnormal spacing below the smallest
normal binade), or by the excess over the largest finite value where it saturates. The bounds
below are exactly that, times the scale, plus 2^-21 |h| for the fp32 roundings of the scaling
and of the decode. At a midpoint between two grid values the error reaches the bound.

Encoding here is done by nearest-neighbour search over the table of representable magnitudes
(ties to the even code), deliberately unlike the bit arithmetic of the device encoder.
The sign bit of a code is the sign bit of its fp32 input.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def e4m3_value_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (OCP 8-bit FP spec, E4M3 variant); NaN for 0x7F/0xFF."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e2m1_value_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes (OCP Microscaling spec, FP4 E2M1)."""
    vals = np.empty(16, dtype=np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        vals[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


E4M3 = e4m3_value_table()
E2M1 = e2m1_value_table()
E4M3_MAX_CODE = 0x7E  # 448
E2M1_MAX_CODE = 0x7   # 6
SCALE_FLOOR_FP8 = F32(2.0 ** -126)       # smallest normal fp32
SCALE_FLOOR_FP4_TILE = F32(2.0 ** -117)  # 2^-126 / 2^-9 (smallest E4M3 subnormal)


def _encode_nearest(v: np.ndarray, mags: np.ndarray, sign_bit: int) -> np.ndarray:
    """Round-to-nearest-even onto a monotone table of non-negative magnitudes (code = index),
    saturating at the last entry."""
    v = np.asarray(v, dtype=F32)
    neg = np.signbit(v)
    a = np.abs(v).astype(np.float64)  # exact
    top = len(mags) - 1
    idx = np.searchsorted(mags, a, side="left")  # mags[idx-1] < a <= mags[idx]
    idx = np.clip(idx, 1, top)
    lo, hi = mags[idx - 1], mags[idx]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((idx % 2) == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(a >= mags[top], top, code)
    code = np.where(a <= mags[0], 0, code)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def e4m3_encode(v) -> np.ndarray:
    return _encode_nearest(v, E4M3[:E4M3_MAX_CODE + 1], 0x80)


def e2m1_encode(v) -> np.ndarray:
    return _encode_nearest(v, E2M1[:E2M1_MAX_CODE + 1], 0x8)


def e4m3_decode(c) -> np.ndarray:
    return E4M3[np.asarray(c, dtype=np.int64)].astype(F32)


def e2m1_decode(c) -> np.ndarray:
    return E2M1[np.asarray(c, dtype=np.int64)].astype(F32)


# ----------------------------------------------------------------------------------------------
# fp8 row copy
# ----------------------------------------------------------------------------------------------
def fp8_row_quantize(h: np.ndarray):
    """h fp32 [..., P, N] -> (codes u8 [..., P, N], scale fp32 [..., P])."""
    h = np.asarray(h, dtype=F32)
    amax = np.max(np.abs(h), axis=-1)
    s = np.where(amax > 0, np.maximum(amax / F32(448.0), SCALE_FLOOR_FP8), F32(1.0)).astype(F32)
    inv = (F32(1.0) / s).astype(F32)
    codes = e4m3_encode((h * inv[..., None]).astype(F32))
    return codes, s


def fp8_row_decode(codes, s) -> np.ndarray:
    return (e4m3_decode(codes) * np.asarray(s, dtype=F32)[..., None]).astype(F32)


def _half_spacing(v, emin: int, mbits: int) -> np.ndarray:
    """Half the grid spacing of a binary floating-point format with mbits stored mantissa bits
    and smallest normal exponent emin, at the (non-negative, fp64) magnitude v: 2^(e - mbits - 1)
    with e = floor(log2 v), and e = emin for subnormal v (the spacing is constant there)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(np.where(v > 0, e, emin), emin)
    return np.exp2(e - mbits - 1)


def fp8_row_bound(h, s) -> np.ndarray:
    """Elementwise |Q(h) - h| bound for the fp8 row copy with row scales s: half the E4M3 grid
    spacing at v = |h|/s (2^(floor(log2 v) - 4), 2^-10 in the subnormal range), or the excess over
    448 s where the code saturates, times s; plus 2^-21 |h| for the fp32 roundings."""
    a = np.abs(np.asarray(h, dtype=np.float64))
    s = np.broadcast_to(np.asarray(s, dtype=np.float64)[..., None], a.shape)
    half = _half_spacing(a / s, -6, 3) * s
    return np.maximum(half, a - 448.0 * s) + 2.0 ** -21 * a


# ----------------------------------------------------------------------------------------------
# fp4 block copy (NVFP4 reading)
# ----------------------------------------------------------------------------------------------
def fp4_quantize(h: np.ndarray):
    """h fp32 [..., P, N] (N % 16 == 0) -> (codes u8 [..., P, N] (one e2m1 code per element),
    block-scale codes u8 [..., P, N/16], tile scale fp32 [...])."""
    h = np.asarray(h, dtype=F32)
    P, N = h.shape[-2:]
    amax_t = np.max(np.abs(h), axis=(-2, -1))
    s_t = np.where(amax_t > 0, np.maximum(amax_t / F32(2688.0), SCALE_FLOOR_FP4_TILE),
                   F32(1.0)).astype(F32)
    d = (F32(6.0) * s_t).astype(F32)
    blk = h.reshape(h.shape[:-1] + (N // 16, 16))
    amax_b = np.max(np.abs(blk), axis=-1)
    r = (amax_b / d[..., None, None]).astype(F32)
    sb_code = e4m3_encode(r)
    s_b = e4m3_decode(sb_code)
    S = (s_b * s_t[..., None, None]).astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(S > 0, F32(1.0) / S, F32(0.0)).astype(F32)
    codes = e2m1_encode((blk * inv[..., None]).astype(F32))
    codes = np.where((S > 0)[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(h.shape), sb_code, s_t


def fp4_scales(sb_code, s_t) -> np.ndarray:
    """Effective per-block scale S = s_b * s_t (fp32) [..., P, N/16]."""
    return (e4m3_decode(sb_code) * np.asarray(s_t, dtype=F32)[..., None, None]).astype(F32)


def fp4_decode(codes, sb_code, s_t) -> np.ndarray:
    S = fp4_scales(sb_code, s_t)
    c = np.asarray(codes)
    P, N = c.shape[-2:]
    v = e2m1_decode(c).reshape(c.shape[:-1] + (N // 16, 16))
    return (v * S[..., None]).astype(F32).reshape(c.shape)


def fp4_bound(h, S) -> np.ndarray:
    """Elementwise |Q(h) - h| bound for the fp4 copy with effective block scales S [..., P, N/16]:
    half the E2M1 grid spacing at v = |h|/S (2^(floor(log2 v) - 2), 1/4 below 1), or the excess
    over 6 S where the code saturates, times S; |h| itself where S == 0 (the block decodes to 0);
    plus 2^-21 |h| for the fp32 roundings."""
    a = np.abs(np.asarray(h, dtype=np.float64))
    Sx = np.repeat(np.asarray(S, dtype=np.float64), 16, axis=-1)
    pos = Sx > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(pos, a / np.where(pos, Sx, 1.0), 0.0)
    half = _half_spacing(v, 0, 1) * Sx
    bnd = np.where(pos, np.maximum(half, a - 6.0 * Sx), a)
    return bnd + 2.0 ** -21 * a


def output_bound(bnd, c, decay=1.0) -> np.ndarray:
    """Bound on the change of the row products y[p] = decay * sum_n h[p, n] c[n] when h is replaced
    by its copy: decay * sum_n bnd[p, n] |c[n]| (triangle inequality; reached when every term's
    error has the sign of c[n]). bnd [..., P, N], c [..., N], decay scalar or [...]."""
    bnd = np.asarray(bnd, dtype=np.float64)
    c = np.abs(np.asarray(c, dtype=np.float64))
    return np.asarray(decay, dtype=np.float64)[..., None] * np.einsum("...pn,...n->...p", bnd, c)
