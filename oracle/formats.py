"""Number formats used by NVFP4, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

* E2M1 (4-bit float, 1 sign, 2 exponent, 1 mantissa bit): the magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6, largest value 6 [QeRL summary, §3.4,
  "Floating-point quantization and NVFP4's E2M1 format"].  Code bit 3 is
  the sign, bits 2..0 index the magnitude list in increasing order.
* E4M3 block scales [QeRL summary, §3.4, Eq. 6: "block-wise scalers stored
  in FP8 (E4M3)"].  The bit layout is the OCP 8-bit floating point
  specification's E4M3 ("FN") encoding, which the pages do not spell out:
  exponent bias 7, no infinities, exponent field 15 with mantissa 7 is
  NaN, largest finite value 448, smallest subnormal 2**-9.
* bf16 (inputs) and fp32 (the per-tensor scale S_FP32).

Everything here is exact: values are Python floats that are exactly the
format's values, and rounding is done by exact comparisons with
``fractions.Fraction`` or with fp64 products that are provably exact.
"""
from fractions import Fraction

import numpy as np

# E2M1 magnitudes, code 0..7 [QeRL summary, §3.4, E2M1 level list].
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_MAX = 6.0


def e4m3_decode(code):
    """Value of a non-negative OCP E4M3FN code 0..126 (127 is NaN)."""
    code = int(code)
    if not 0 <= code <= 126:
        raise ValueError("E4M3 code out of the finite non-negative range")
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9              # subnormal: m/8 * 2**(1-7)
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


# All non-negative finite E4M3 values, index == code, strictly increasing.
E4M3_VALUES = np.array([e4m3_decode(c) for c in range(127)], dtype=np.float64)
E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_bits(x):
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def round_fraction_to_f32(q):
    """Round an exact non-negative rational to the nearest fp32, ties to even.

    Written from the IEEE 754 definition of round-to-nearest-even: pick the
    representable neighbours below and above q and compare distances in
    exact arithmetic.  Overflow saturates to +inf like IEEE rounding.
    """
    q = Fraction(q)
    if q < 0:
        raise ValueError("non-negative input expected")
    if q == 0:
        return np.float32(0.0)
    guess = np.float32(float(q))          # within an ulp or two of q
    cands = {guess}
    for _ in range(2):
        nxt = set()
        for c in cands:
            nxt.add(np.nextafter(c, np.float32(0)))
            nxt.add(np.nextafter(c, np.float32(np.inf)))
        cands |= nxt
    cands = sorted(c for c in cands if np.isfinite(c) and c >= 0)
    below = max((c for c in cands if Fraction(float(c)) <= q), default=None)
    above = min((c for c in cands if Fraction(float(c)) >= q), default=None)
    if above is None:
        return np.float32(np.inf)
    if below is None:
        return above
    if below == above:
        return below
    db, da = q - Fraction(float(below)), Fraction(float(above)) - q
    if db < da:
        return below
    if da < db:
        return above
    return below if (f32_bits(below) & 1) == 0 else above


def rne_index_on_grid(values, grid):
    """Round each value to the nearest point of a sorted grid, ties to the
    even index, saturating at both ends.

    ``grid`` is a 1-D increasing array (grid[0] >= 0).  The index returned
    is the number of midpoints the value lies above, where a value exactly
    on a midpoint between index i and i+1 goes to whichever of i, i+1 is
    even.  Callers guarantee that grid values, midpoints and ``values`` are
    exact fp64 numbers, so every comparison is exact.
    """
    values = np.asarray(values, dtype=np.float64)
    grid = np.asarray(grid, dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) * 0.5
    lo = np.searchsorted(mids, values, side="left")    # midpoints < v
    hi = np.searchsorted(mids, values, side="right")   # midpoints <= v
    tie = hi > lo
    idx = lo + (tie & (lo % 2 == 1))
    return idx.astype(np.int64)
