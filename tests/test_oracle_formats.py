"""Pins for the oracle's element formats and RTN encoders (CPU).

The checks come from outside the oracle: closed-form value sets of the OCP
E2M1 / E4M3-FN formats, and exact rational brute force of round-to-nearest
with ties to the even code.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats


def test_e2m1_value_set_closed_form():
    mags = sorted({abs(formats.e2m1_value(c)) for c in range(16)})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert formats.e2m1_value(c) == -formats.e2m1_value(c | 8)
    assert np.signbit(formats.E2M1_VALUES[8])  # code 0x8 is negative zero
    # codes 0..7 are increasing
    assert np.all(np.diff(formats.E2M1_VALUES[:8]) > 0)


def test_e4m3_closed_form_landmarks():
    v = formats.E4M3_VALUES
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0  # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0xB8] == -1.0
    finite_nonneg = v[:0x7F]
    assert len(finite_nonneg) == 127
    assert np.all(np.diff(finite_nonneg) > 0)
    # every normal value has at most 4 significant bits
    for b in range(0x08, 0x7F):
        m, e = np.frexp(v[b])
        assert (m * 16) == int(m * 16)


def _brute_rne(mag: Fraction, grid, codes):
    """Nearest grid point by exact rational distance; ties to the even code; saturate."""
    if mag >= grid[-1]:
        return codes[-1]
    best = None
    for g, c in zip(grid, codes):
        d = abs(mag - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def _brute_rne_vec(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Vectorized brute force: argmin of |v - g| over all grid points, ties to the even code.

    Valid where every distance is exact in float64 (float32 inputs of moderate
    exponent against grid points with <= 4 significant bits)."""
    d = np.abs(v.astype(np.float64)[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    codes = np.arange(len(grid))
    even = cand & (codes[None, :] % 2 == 0)
    pick_even = even.any(axis=1)
    first = np.argmax(cand, axis=1)
    first_even = np.argmax(even, axis=1)
    out = np.where(pick_even, first_even, first)
    return np.where(v >= grid[-1], len(grid) - 1, out)


def test_e2m1_encoder_exhaustive_bf16_times_scales():
    """Every finite BF16 magnitude times several multipliers: encoder == brute-force argmin."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # all finite non-negative bf16
    base = (bits << 16).view(np.float32)
    for mult in (np.float32(1.0), np.float32(0.8), np.float32(3.0), np.float32(2.0 ** 20)):
        with np.errstate(over="ignore"):
            vals = (base * mult).astype(np.float32)
        vals = vals[np.isfinite(vals)]
        # distances are exact in float64 for magnitudes in [2^-20, 2^20]
        vals = vals[(vals > 2.0 ** -20) & (vals < 2.0 ** 20)]
        got = formats.e2m1_encode(vals).astype(np.int64)
        want = _brute_rne_vec(vals, formats.E2M1_GRID)
        assert np.array_equal(got, want)
        gotn = formats.e2m1_encode(-vals).astype(np.int64)
        assert np.array_equal(gotn, want | 8)
    # every exact midpoint and its float32 neighbours, against exact rationals
    grid = [Fraction(float(g)) for g in formats.E2M1_GRID]
    codes = list(range(8))
    for a, b in zip(formats.E2M1_GRID[:-1], formats.E2M1_GRID[1:]):
        mid = np.float32((a + b) / 2)
        for v in (np.nextafter(mid, np.float32(0)), mid, np.nextafter(mid, np.float32(10))):
            got = int(formats.e2m1_encode(np.array([v], dtype=np.float32))[0])
            assert got == _brute_rne(Fraction(float(v)), grid, codes)
            gotn = int(formats.e2m1_encode(np.array([-v], dtype=np.float32))[0])
            assert gotn == got | 8
    assert int(formats.e2m1_encode(np.array([1e30], np.float32))[0]) == 7
    assert int(formats.e2m1_encode(np.array([-0.0], np.float32))[0]) == 8
    assert int(formats.e2m1_encode(np.array([0.0], np.float32))[0]) == 0


def test_e4m3_encoder_midpoints_and_neighbours():
    grid = [Fraction(float(g)) for g in formats.E4M3_GRID]
    codes = list(range(0x7F))
    pts = []
    for a, b in zip(formats.E4M3_GRID[:-1], formats.E4M3_GRID[1:]):
        mid = np.float32((a + b) / 2)
        pts += [np.nextafter(mid, np.float32(0)), mid, np.nextafter(mid, np.float32(1e9)), np.float32(a)]
    pts += [np.float32(448.0), np.float32(464.0), np.float32(480.0), np.float32(1e6), np.float32(2.0 ** -11),
            np.float32(2.0 ** -10), np.float32(0.0)]
    pts = np.array(pts, dtype=np.float32)
    got = formats.e4m3_encode_nonneg(pts)
    for v, c in zip(pts, got):
        assert int(c) == _brute_rne(Fraction(float(v)), grid, codes), float(v)
    # spot values fixed by the definition
    enc = lambda s: int(formats.e4m3_encode_nonneg(np.array([s], np.float32))[0])  # noqa: E731
    assert enc(1.0) == 0x38
    assert enc(1.0625) == 0x38  # tie between 0x38 and 0x39 -> even
    assert enc(1.1875) == 0x3A  # tie between 0x39 and 0x3A -> even
    assert enc(2.0 ** -10) == 0x00  # tie between 0 and the smallest subnormal -> even (zero)
    assert enc(1.5 * 2.0 ** -9) == 0x02  # tie between 0x01 and 0x02 -> even
    assert enc(1e9) == 0x7E


def test_encoders_reject_negative_magnitudes():
    with pytest.raises(ValueError):
        formats.round_to_grid_rne(np.array([-1.0]), formats.E2M1_GRID, formats.E2M1_GRID_CODES)
