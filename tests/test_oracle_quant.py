"""Pins of the read-copy quantizer emulation (CPU only).

Code tables are pinned to the OCP format definitions (hand-written golden points in tests/golden)
and to torch's float8_e4m3fn (a library implementation of OCP E4M3); rounding is pinned to
brute-force nearest-value search with ties to even; the error bounds are checked for soundness on
random and adversarial tiles.
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
