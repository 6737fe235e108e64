"""Pins of the oracle's number formats (bf16, E4M3FN, E2M1) against their
definitions, hand-derived rounding cases and torch's independent casts."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle.codecs import (E2M1_VALUES, bf16_to_f64, e2m1_decode, e2m1_encode, e4m3_decode,
                           e4m3_encode, f64_to_bf16)


def test_e2m1_grid_golden():
    rows = read_golden("e2m1_grid.txt")
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows])
    got = e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16)
    assert np.array_equal(e2m1_encode(e2m1_decode(codes)), codes)


def test_e2m1_rounding_golden():
    rows = read_golden("e2m1_rounding.txt")
    x = np.array([float(r[0]) for r in rows])
    want = np.array([int(r[1]) for r in rows])
    assert np.array_equal(e2m1_encode(x), want)


def _nearest_even(x, grid_vals, grid_codes):
    """Brute force: nearest grid value by distance; equal distances -> even code."""
    out = []
    for v in x:
        a = abs(v)
        best = None
        for val, code in zip(grid_vals, grid_codes):
            dist = abs(a - val)
            key = (dist, code & 1)
            if best is None or key < best[0]:
                best = (key, code)
        out.append(best[1] | (8 if np.signbit(v) else 0))
    return np.array(out)


def test_e2m1_bruteforce():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-7, 7, 3000).astype(np.float32).astype(np.float64),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5]),
                        -np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])])
    # saturation: beyond 6 the nearest grid value is 6 anyway, so brute force applies directly
    want = _nearest_even(x, E2M1_VALUES, list(range(8)))
    assert np.array_equal(e2m1_encode(x), want)


def test_e4m3_golden():
    rows = read_golden("e4m3_points.txt")
    x = np.array([float(r[0]) for r in rows])
    want = np.array([int(r[1], 16) for r in rows])
    assert np.array_equal(e4m3_encode(x), want)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()
    finite = e4m3_decode(np.arange(0x7F))
    assert finite.max() == 448.0 and finite[1] == 2.0 ** -9 and np.all(np.diff(finite) > 0)


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(5)
    grid = e4m3_decode(np.arange(0x7F))
    mids = (grid[1:] + grid[:-1]) / 2            # every tie point
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000)),
        mids, -mids, grid, -grid, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    x = x[np.abs(x) <= 464].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_e4m3_saturates_instead_of_nan():
    x = np.array([465.0, 480.0, 1e30, -470.0])
    assert np.array_equal(e4m3_encode(x), [0x7E, 0x7E, 0x7E, 0xFE])


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x32 = np.concatenate([rng.standard_normal(50000).astype(np.float32),
                          (rng.standard_normal(2000) * 1e-39).astype(np.float32),
                          np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], dtype=np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16(x32.astype(np.float64)), ref)
    assert np.array_equal(bf16_to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_bf16_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30 is just above the midpoint of 1 and 1+2^-7: one rounding gives 1+2^-7,
    # a detour through float32 would give the tie and then 1.0
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_to_f64(f64_to_bf16(np.array([x])))[0] == 1.0 + 2.0 ** -7
