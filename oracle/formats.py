"""FP4 E2M1 and FP8 E4M3 ("FN") element formats, written from their bit layouts.

The "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, section "Quantization
Setup", names the formats: weights FP4 E2M1, block scales FP8 E4M3.  The pages
only name them; the bit-level meaning below is the public OCP 8-bit floating
point / microscaling definition of those two formats:

* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  exponent field 0 is subnormal: magnitude = 0.5 * m;
  otherwise magnitude = 2**(e - 1) * (1 + m / 2).
* E4M3 "FN": 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no inf;
  the all-ones pattern S.1111.111 is NaN, so the largest finite value is
  S.1111.110 = 448.  exponent field 0 is subnormal: magnitude = 2**-6 * m / 8;
  otherwise magnitude = 2**(e - 7) * (1 + m / 8).

Rounding is round-to-nearest ("standard NVFP4 PTQ (RTN)", same section).  The
tie rule is not on the pages; the reading taken is ties-to-even on the code,
and saturation to the largest finite magnitude (no inf exists in either
format).  Both encoders here are the generic "nearest element of a finite,
sorted value set" rule, applied to each format's value table.

Everything here is TEST INFRASTRUCTURE for checking the HIP path.
"""

from __future__ import annotations

import numpy as np


def e2m1_magnitude(code: int) -> float:
    """Magnitude of an E2M1 code's low 3 bits (exponent e = bits 2:1, mantissa m = bit 0)."""
    c = code & 0x7
    e, m = c >> 1, c & 1
    if e == 0:
        return 0.5 * m
    return 2.0 ** (e - 1) * (1.0 + m / 2.0)


def e2m1_value(code: int) -> float:
    """Signed value of a 4-bit E2M1 code (bit 3 is the sign)."""
    mag = e2m1_magnitude(code)
    return -mag if (code & 0x8) else mag


def e4m3_value(byte: int) -> float:
    """Signed value of an E4M3 "FN" byte; NaN for the two all-ones patterns."""
    s, e, m = (byte >> 7) & 1, (byte >> 3) & 0xF, byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = 2.0 ** -6 * (m / 8.0)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


# Value tables: code -> value, as float64 arrays (all values are exact in fp64).
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_VALUES = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)

# Non-negative finite grids sorted by value, with the code of each grid point.
# For both formats the non-negative codes are already ordered by value
# (exponent field above mantissa field), so code i is the i-th grid point.
E2M1_GRID_CODES = np.arange(8, dtype=np.int64)
E2M1_GRID = E2M1_VALUES[:8].copy()
E4M3_GRID_CODES = np.arange(0x7F, dtype=np.int64)  # 0x00 .. 0x7E; 0x7F is NaN
E4M3_GRID = E4M3_VALUES[:0x7F].copy()


def round_to_grid_rne(mag: np.ndarray, grid: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Round non-negative magnitudes to the nearest point of a sorted finite grid.

    * exact ties between two neighbouring grid points go to the even code;
    * magnitudes beyond the last grid point saturate to it (the formats have no
      infinity, and saturation is the reading taken for an overflowing RTN).

    The decision compares ``mag`` against the exact midpoint of the two grid
    neighbours.  Grid points have at most 4 significant bits, so each midpoint
    is exact in float64, and so is every float32 input: the comparison is exact.
    """
    mag = np.asarray(mag, dtype=np.float64)
    if np.any(mag < 0) or np.any(np.isnan(mag)):
        raise ValueError("round_to_grid_rne expects non-negative, non-NaN magnitudes")
    hi = np.searchsorted(grid, mag, side="left")  # grid[hi-1] < mag <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    g_lo, g_hi = grid[lo], grid[hi]
    mid = (g_lo + g_hi) / 2.0
    pick_hi = mag > mid
    tie = mag == mid
    hi_even = (codes[hi] & 1) == 0
    pick_hi = np.where(tie, hi_even, pick_hi)
    out = np.where(pick_hi, codes[hi], codes[lo])
    # below the first grid point (only possible if grid[0] > 0) -> first point
    out = np.where(mag <= grid[0], codes[0], out)
    # beyond the last grid point -> saturate
    out = np.where(mag >= grid[-1], codes[-1], out)
    return out.astype(np.int64)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """E2M1 RTN-even with saturation at 6; sign bit = signbit(v) (so -0.0 -> 0x8)."""
    v = np.asarray(v, dtype=np.float64)
    mag_code = round_to_grid_rne(np.abs(v), E2M1_GRID, E2M1_GRID_CODES)
    sign = np.signbit(v).astype(np.int64)
    return (mag_code | (sign << 3)).astype(np.uint8)


def e4m3_encode_nonneg(s: np.ndarray) -> np.ndarray:
    """E4M3 RTN-even for a non-negative scale, saturating at 448 (code 0x7E)."""
    return round_to_grid_rne(np.asarray(s, dtype=np.float64), E4M3_GRID, E4M3_GRID_CODES).astype(np.uint8)
