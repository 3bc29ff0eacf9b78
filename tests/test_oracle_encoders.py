"""Pins for the oracle's number-format encoders (CPU only).

The oracle writes bf16, E4M3FN and UE8M0 conversions from the format
definitions. Here they are checked against (a) hand-derived points of those
definitions under tests/golden/, (b) torch's CPU casts, exhaustively over every
bf16 input and over random binary32 inputs, and (c) the defining inequality of
the round-up power-of-two scale, in exact rational arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_points(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parts[0], int(parts[1], 16)))
    return rows


def test_e4m3_golden_points(orc):
    pts = _read_points("e4m3fn_points.txt")
    vals = np.array([float(v) for v, _ in pts], dtype=np.float32)
    want = np.array([c for _, c in pts], dtype=np.uint8)
    got = orc.f32_to_e4m3(vals)
    bad = [(pts[i][0], hex(got[i]), hex(want[i])) for i in range(len(pts))
           if got[i] != want[i]]
    assert not bad, bad


def test_bf16_golden_points(orc):
    pts = _read_points("bf16_points.txt")
    bits = np.array([int(v, 16) for v, _ in pts], dtype=np.uint32)
    want = np.array([c for _, c in pts], dtype=np.uint16)
    got = orc.f32_to_bf16(bits.view(np.float32))
    assert np.array_equal(got, want), (got, want)


def _torch_bf16_bits(f32):
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_random(orc):
    g = np.random.default_rng(1)
    bits = g.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties
    bits[:200_000] = (bits[:200_000] & 0xFFFF0000) | 0x8000
    bits[200_000:300_000] = (bits[200_000:300_000] & 0xFFFF0000) | 0x7FFF
    f = bits.view(np.float32)
    finite = ~np.isnan(f)
    got = orc.f32_to_bf16(f)
    want = _torch_bf16_bits(f.copy())
    assert np.array_equal(got[finite], want[finite])
    # NaN stays NaN
    assert np.all(np.isnan(orc.bf16_to_f32(got[~finite])))


def _all_bf16_finite():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (h.astype(np.uint32) << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("scale", [1.0, 0.125, 3.7, 1e-3, 97.0, 2.0**-12])
def test_e4m3_matches_torch_exhaustive_bf16(orc, scale):
    """Every finite bf16 value times a scale, clamped to +-448, against torch's
    float8_e4m3fn cast (round to nearest even)."""
    f = _all_bf16_finite() * np.float32(scale)
    f = np.clip(f, -448.0, 448.0).astype(np.float32)
    got = orc.f32_to_e4m3(f)
    want = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_matches_torch_random_f32(orc):
    g = np.random.default_rng(2)
    f = (g.uniform(-1.0, 1.0, size=3_000_000) *
         np.exp2(g.integers(-14, 9, size=3_000_000))).astype(np.float32)
    f = np.clip(f, -448.0, 448.0)
    got = orc.f32_to_e4m3(f)
    want = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_saturates_and_nan(orc):
    f = np.array([449.0, 479.0, 480.0, 1e6, np.inf, -1e6, -np.inf, np.nan],
                 dtype=np.float32)
    got = orc.f32_to_e4m3(f)
    assert list(got[:7]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[7] == 0x7F


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_to_f32(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_widen_is_exact(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    want = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ---------------------------------------------------------------- UE8M0
INV448 = np.float32(1.0) / np.float32(448.0)


def _p(amax):
    return Fraction(float(np.float32(amax) * INV448))


def test_ue8m0_crafted_blocks(orc):
    """amax = 448 * 2^j maps to 127 + j; just above moves up one; just below
    stays; zero gives byte 0."""
    js = np.arange(-20, 20)
    exact = (448.0 * np.exp2(js)).astype(np.float32)
    assert np.array_equal(orc.ue8m0_from_amax(exact), (127 + js).astype(np.uint8))
    above = (exact * np.float32(1 + 2.0**-8)).astype(np.float32)
    assert np.array_equal(orc.ue8m0_from_amax(above), (128 + js).astype(np.uint8))
    below = (exact * np.float32(1 - 2.0**-8)).astype(np.float32)
    assert np.array_equal(orc.ue8m0_from_amax(below), (127 + js).astype(np.uint8))
    assert orc.ue8m0_from_amax(np.array([0.0], np.float32))[0] == 0


def test_ue8m0_is_smallest_power_at_or_above(orc):
    """byte - 127 is the least integer n with 2^n >= amax * (1/448) (in fp32),
    checked in exact rational arithmetic; clamped to [0, 254]."""
    g = np.random.default_rng(3)
    # every positive finite bf16 magnitude, plus random fp32 values
    bf = _all_bf16_finite()
    amax = np.concatenate([bf[bf > 0], np.abs(g.standard_normal(20000)).astype(np.float32)])
    got = orc.ue8m0_from_amax(amax.astype(np.float32))
    for a, b in zip(amax[::7], got[::7]):
        p = _p(a)
        n = int(b) - 127
        if 0 < b < 254:
            assert Fraction(2) ** n >= p and Fraction(2) ** (n - 1) < p, (a, b)
        elif b == 0:
            assert Fraction(2) ** -127 >= p
        else:
            assert Fraction(2) ** 127 < p or Fraction(2) ** 127 >= p


def test_ue8m0_never_overflows_e4m3(orc):
    """With the round-up scale, the block max times 2^(127-byte) is <= 448
    (up to the rounding of the fp32 product)."""
    bf = _all_bf16_finite()
    amax = bf[(bf > 1e-30) & (bf < 1e30)]
    b = orc.ue8m0_from_amax(amax).astype(np.int64)
    scaled = amax.astype(np.float64) * np.exp2(127 - b)
    assert np.all(scaled <= 448.0 * (1 + 2.0**-22))
    assert np.all(scaled > 224.0 * (1 - 2.0**-22))
    assert math.isfinite(float(scaled.max()))
