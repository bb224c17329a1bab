"""Pins of the read-copy quantizer emulation (CPU only).

Code tables are pinned to the OCP format definitions (hand-written golden points in tests/golden)
and to torch's float8_e4m3fn (a library implementation of OCP E4M3); rounding is pinned to
brute-force nearest-value search with ties to even; the error bounds are checked for soundness on
random and adversarial tiles and for tightness at inputs where the rounding error must reach them
(midpoints between grid values, the subnormal range, saturation, a zero block scale); the scale
floors are checked on tiles too small for an unfloored scale to have a finite reciprocal.
"""
import os

import numpy as np
import pytest
import torch

from oracle import quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_points(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()[:2]
            rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_table_matches_ocp_definition():
    pts = _read_points("ocp_e2m1_values.txt")
    assert len(pts) == 16
    for c, v in pts:
        assert quant.E2M1[c] == v and np.signbit(quant.E2M1[c]) == np.signbit(v)


def test_e4m3_named_points_match_ocp_definition():
    for c, v in _read_points("ocp_e4m3_points.txt"):
        if np.isnan(v):
            assert np.isnan(quant.E4M3[c])
        else:
            assert quant.E4M3[c] == v and np.signbit(quant.E4M3[c]) == np.signbit(v)


def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(quant.E4M3)
    assert np.all(both_nan | (ref == quant.E4M3))
    assert both_nan.sum() == 2


def test_round_trip_all_codes():
    for c in range(256):
        if np.isnan(quant.E4M3[c]):
            continue
        assert quant.e4m3_encode(np.float32(quant.E4M3[c]))[()] == c
    for c in range(16):
        assert quant.e2m1_encode(np.float32(quant.E2M1[c]))[()] == c


def _brute_force(v, table, max_code, sign_bit):
    """Nearest finite magnitude, ties to the even code, saturating."""
    a = abs(float(v))
    best = None
    for c in range(max_code + 1):
        d = abs(table[c] - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    return c | (sign_bit if np.signbit(np.float32(v)) else 0)


def test_encode_matches_brute_force_including_ties():
    rng = np.random.default_rng(0)
    mags = quant.E4M3[:quant.E4M3_MAX_CODE + 1]
    mids = (mags[1:] + mags[:-1]) / 2  # exact ties
    vals = np.concatenate([rng.standard_normal(3000) * 50, mids, -mids, [0.0, 447.9, 448.0, 449.0,
                           464.0, 480.0, 1e6, -1e6, 1e-6, 2.0 ** -10, 3 * 2.0 ** -11]])
    vals = vals.astype(np.float32)
    got = quant.e4m3_encode(vals)
    for v, c in zip(vals, got):
        assert c == _brute_force(v, quant.E4M3, quant.E4M3_MAX_CODE, 0x80), v
    m2 = quant.E2M1[:8]
    vals = np.concatenate([rng.standard_normal(2000) * 4, (m2[1:] + m2[:-1]) / 2, [7.0, -100.0]])
    vals = vals.astype(np.float32)
    got = quant.e2m1_encode(vals)
    for v, c in zip(vals, got):
        assert c == _brute_force(v, quant.E2M1, quant.E2M1_MAX_CODE, 0x8), v


def test_in_range_encode_matches_torch_cast():
    # torch's float8_e4m3fn cast is round-to-nearest-even; inside +-448 it must agree bit for bit
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 30, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(quant.e4m3_encode(v), ref)


def test_fp8_row_scale_definition():
    rng = np.random.default_rng(2)
    h = (rng.standard_normal((3, 4, 32)) * 0.3).astype(np.float32)
    h[1, 2] = 0.0
    codes, s = quant.fp8_row_quantize(h)
    assert s.dtype == np.float32
    assert s[1, 2] == 1.0 and np.all(codes[1, 2] == 0)
    # the row maximum maps to +-448 (code 0x7E / 0xFE)
    am = np.abs(h).argmax(-1)
    top = np.take_along_axis(codes, am[..., None], -1)[..., 0]
    mask = np.ones_like(top, dtype=bool)
    mask[1, 2] = False
    assert np.all((top[mask] & 0x7F) == 0x7E)


def _adversarial_tiles(rng):
    tiles = [rng.standard_normal((8, 64)).astype(np.float32) * 0.3]
    t = rng.standard_normal((8, 64)).astype(np.float32) * 1e-3
    t[3, 5] = 50.0  # one huge element: everything else falls in the subnormal range
    tiles.append(t)
    t = np.zeros((8, 64), np.float32)
    t[0, :16] = 1e-30  # a block whose scale underflows to zero
    t[5, 7] = 2.0
    tiles.append(t)
    tiles.append(np.zeros((8, 64), np.float32))
    tiles.append((rng.standard_cauchy((8, 64)) * 0.1).astype(np.float32))
    return tiles


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_bound_is_sound(seed):
    rng = np.random.default_rng(seed)
    for h in _adversarial_tiles(rng):
        codes, s = quant.fp8_row_quantize(h)
        err = np.abs(quant.fp8_row_decode(codes, s).astype(np.float64) - h)
        assert np.all(err <= quant.fp8_row_bound(h, s))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp4_bound_is_sound(seed):
    rng = np.random.default_rng(seed)
    for h in _adversarial_tiles(rng):
        codes, sb, st = quant.fp4_quantize(h)
        S = quant.fp4_scales(sb, st)
        err = np.abs(quant.fp4_decode(codes, sb, st).astype(np.float64) - h)
        assert np.all(err <= quant.fp4_bound(h, S))


def test_fp4_two_level_scale_definition():
    rng = np.random.default_rng(3)
    h = (rng.standard_normal((2, 16, 64)) * 0.3).astype(np.float32)
    codes, sb, st = quant.fp4_quantize(h)
    amax = np.abs(h).max(axis=(1, 2))
    np.testing.assert_array_equal(st, (amax / np.float32(2688)).astype(np.float32))
    # the block holding the tile maximum gets block scale 448 and the maximum maps to +-6
    for i in range(2):
        p, n = np.unravel_index(np.abs(h[i]).argmax(), h[i].shape)
        assert sb[i, p, n // 16] == 0x7E
        assert codes[i, p, n] & 0x7 == 0x7


# ----------------------------------------------------------------------------------------------
# Tightness of the bounds: inputs at exact midpoints between grid values (ties to even), in the
# subnormal range and past saturation, where the rounding error must reach the bound. A bound
# that a slip loosened (a wrong power of two, 0.5 for 0.25, a dropped scale) fails here; one
# that it tightened fails the soundness tests above.
# ----------------------------------------------------------------------------------------------
TIGHT = 0.99  # the error reaches the bound up to the 2^-21 |h| term for the fp32 roundings


def _fp8_tight_row():
    """One row with amax 448 (scale exactly 1), so every other element is its own scaled value:
    midpoints just above each power of two 2^e (1 + 1/16), between the two lowest normal values,
    and in the subnormal range."""
    v = [448.0]
    v += [2.0 ** e * (1 + 1 / 16) for e in range(-6, 8)]       # tie -> 2^e (even mantissa 0)
    v += [2.0 ** e * (1 + 3 / 16) for e in range(-6, 8)]       # tie -> 2^e (1 + 1/4) (even)
    v += [2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 13 * 2.0 ** -10]  # subnormal midpoints
    v += [-x for x in v[1:8]]
    row = np.zeros(64, np.float32)
    row[:len(v)] = v
    return row, len(v)


def test_fp8_bound_is_tight_at_midpoints():
    row, n = _fp8_tight_row()
    h = row[None, None, :]
    codes, s = quant.fp8_row_quantize(h)
    assert s[0, 0] == 1.0
    err = np.abs(quant.fp8_row_decode(codes, s).astype(np.float64) - h)[0, 0, 1:n]
    bnd = quant.fp8_row_bound(h, s)[0, 0, 1:n]
    assert np.all(err <= bnd)
    assert np.all(err >= TIGHT * bnd), (err / bnd).min()
    # the same row scaled by a power of two (scale 2^-20): the bound scales with it
    h2 = (row * np.float32(2.0 ** -20))[None, None, :]
    c2, s2 = quant.fp8_row_quantize(h2)
    assert s2[0, 0] == np.float32(2.0 ** -20)
    e2 = np.abs(quant.fp8_row_decode(c2, s2).astype(np.float64) - h2)[0, 0, 1:n]
    b2 = quant.fp8_row_bound(h2, s2)[0, 0, 1:n]
    assert np.all(e2 <= b2) and np.all(e2 >= TIGHT * b2)


def test_fp8_bound_saturation_term_is_tight():
    # a scale below amax / 448 (the writer never picks one; the bound still covers it): elements
    # past 448 s saturate and the error is exactly their excess
    h = np.array([[[500.0, 600.0, 1000.0, -700.0] + [0.0] * 60]], np.float32)
    s = np.ones((1, 1), np.float32)
    codes = quant.e4m3_encode(h)  # scale 1: the scaled values are the inputs
    err = np.abs(quant.fp8_row_decode(codes, s).astype(np.float64) - h)[0, 0, :4]
    bnd = quant.fp8_row_bound(h, s)[0, 0, :4]
    np.testing.assert_allclose(err, [52.0, 152.0, 552.0, 252.0])
    assert np.all(err <= bnd) and np.all(err >= TIGHT * bnd)


def _fp4_tight_tile():
    """A 4 x 64 tile with amax 2688 (tile scale exactly 1): block 0 of row 0 holds 2688 (block
    scale 448), block 1 has amax 6 (block scale 1), so its scaled values are the inputs:
    midpoints above each power of two (1.25, 2.5, 5), in the subnormal range (0.25, 0.75) and
    between 1.5 and 2 (1.75); block 2 has amax 6 * 2^-11 (block scale rounds to 0: everything
    decodes to 0)."""
    t = np.zeros((4, 64), np.float32)
    t[0, 0] = 2688.0
    mids = [6.0, 1.25, 2.5, 5.0, 0.25, 0.75, 1.75, -1.25, -2.5, -5.0, -0.25, -0.75, 3.5, -3.5]
    t[0, 16:16 + len(mids)] = mids
    t[1, 32:36] = [6 * 2.0 ** -11, -6 * 2.0 ** -11, 2.0 ** -12, 0.0]
    return t, len(mids)


def test_fp4_bound_is_tight_at_midpoints_and_zero_block_scale():
    t, n = _fp4_tight_tile()
    codes, sb, st = quant.fp4_quantize(t[None])
    assert st[0] == 1.0 and sb[0, 0, 0] == 0x7E and sb[0, 0, 1] == 0x38 and sb[0, 1, 2] == 0
    S = quant.fp4_scales(sb, st)
    err = np.abs(quant.fp4_decode(codes, sb, st).astype(np.float64) - t[None])[0]
    bnd = quant.fp4_bound(t[None], S)[0]
    assert np.all(err <= bnd)
    sel = err[0, 17:16 + n], bnd[0, 17:16 + n]  # the midpoints (block scale 1)
    assert np.all(sel[0] >= TIGHT * sel[1]), (sel[0] / sel[1]).min()
    z = err[1, 32:35], bnd[1, 32:35]  # zero block scale: error = |h| = bound
    np.testing.assert_array_equal(z[0], np.abs(t[1, 32:35]))
    assert np.all(z[0] >= TIGHT * z[1])


def test_fp4_bound_saturation_term_is_tight():
    # a block scale below amax / 6 (the writer rounds it to nearest, so at most 1/16 below):
    # force S = 1 on values past 6 and the error is exactly the excess
    h = np.zeros((1, 1, 16), np.float32)
    h[0, 0, :3] = [9.0, 14.0, -20.0]
    codes = quant.e2m1_encode(h)
    S = np.ones((1, 1, 1), np.float32)
    err = np.abs(quant.e2m1_decode(codes).astype(np.float64) - h)[0, 0, :3]
    bnd = quant.fp4_bound(h, S)[0, 0, :3]
    np.testing.assert_allclose(err, [3.0, 8.0, 14.0])
    assert np.all(err <= bnd) and np.all(err >= TIGHT * bnd)


def test_scale_floors_keep_tiny_tiles_finite():
    # a row / tile whose largest magnitude is far below 448 (2688) * 2^-126: without the floor
    # the scale is subnormal, its reciprocal infinite, and a zero element encodes 0 * inf = NaN
    h = np.zeros((2, 16, 64), np.float32)
    h[0, 0, 0] = 1e-37
    h[0, 0, 1] = -3e-38
    h[0, 3, 5] = 2e-37
    h[1, 2, 17] = 4e-36
    codes, s = quant.fp8_row_quantize(h)
    assert s[0, 0] == np.float32(2.0 ** -126) and s[1, 2] == np.float32(2.0 ** -126)
    assert np.all(s[0, 1] == 1.0)  # all-zero rows keep scale 1
    dec = quant.fp8_row_decode(codes, s)
    assert np.all(np.isfinite(dec)) and np.all(dec[h == 0] == 0)
    assert np.all(np.abs(dec.astype(np.float64) - h) <= quant.fp8_row_bound(h, s))
    c4, sb, st = quant.fp4_quantize(h)
    np.testing.assert_array_equal(st, np.float32(2.0 ** -117))
    d4 = quant.fp4_decode(c4, sb, st)
    assert np.all(np.isfinite(d4)) and np.all(d4[h == 0] == 0)
    S = quant.fp4_scales(sb, st)
    assert np.all((S == 0) | (S >= np.float32(2.0 ** -126)))
    assert np.all(np.abs(d4.astype(np.float64) - h) <= quant.fp4_bound(h, S))
    # just above the floors nothing changes: scale = amax / 448 (2688) exactly as before
    h2 = np.zeros((1, 1, 64), np.float32)
    h2[0, 0, 0] = np.float32(448 * 2.0 ** -120)
    assert quant.fp8_row_quantize(h2)[1][0, 0] == np.float32(2.0 ** -120)


def test_output_bound_is_reached_when_errors_align():
    # |sum_n (Q - h)[p, n] c[n]| <= sum_n bound[p, n] |c[n]|, with equality when every element
    # sits at a midpoint (error = bound) and c[n] has the sign of its error
    row, n = _fp8_tight_row()
    h = np.stack([row, -row])[None]  # [1][2][64]
    codes, s = quant.fp8_row_quantize(h)
    e = quant.fp8_row_decode(codes, s).astype(np.float64) - h
    bnd = quant.fp8_row_bound(h, s)
    c = np.sign(e[0, 0]) * np.linspace(0.5, 2.0, 64)
    lim = quant.output_bound(bnd, c[None], np.array([0.7]))
    dy = 0.7 * np.einsum("pn,n->p", e[0], c)
    assert np.all(np.abs(dy) <= lim[0])
    assert abs(dy[0]) >= TIGHT * lim[0, 0]
