"""Pins for oracle.formats: page-printed E2M1 levels, the OCP E4M3
definition, and exact rounding checked by brute force."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_levels_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_levels.json")))
    assert list(formats.E2M1_MAGNITUDES) == g["magnitudes"]
    assert formats.E2M1_MAX == g["q_max"]


def test_e4m3_table_closed_form():
    v = formats.E4M3_VALUES
    assert len(v) == 127
    assert np.all(np.diff(v) > 0)
    assert v[0] == 0.0
    assert v[1] == 2.0 ** -9            # smallest subnormal
    assert v[7] == 7 * 2.0 ** -9        # largest subnormal
    assert v[8] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0               # exponent field 7 == bias
    assert v[126] == 448.0 == formats.E4M3_MAX
    # every value has at most 4 significant bits
    for x in v[1:]:
        m = Fraction(float(x))
        while m >= 16:
            m /= 2
        while m < 8:
            m *= 2
        assert m.denominator == 1
    with pytest.raises(ValueError):
        formats.e4m3_decode(127)


def test_bf16_decode():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4040, 0x0001, 0x7F7F],
                    dtype=np.uint16)
    v = formats.bf16_bits_to_f64(bits)
    assert v[0] == 0.0 and np.signbit(v[1])
    assert v[2] == 1.0 and v[3] == -1.0 and v[4] == 3.0
    assert v[5] == 2.0 ** -133
    assert v[6] == (2 - 2.0 ** -7) * 2.0 ** 127


def _brute_f32(q):
    """Nearest fp32 to an exact rational by scanning a bit window."""
    q = Fraction(q)
    base = int(np.array(np.float32(float(q)), dtype=np.float32).view(np.uint32))
    best = None
    for b in range(max(0, base - 4), base + 5):
        c = np.array(b, dtype=np.uint32).view(np.float32)
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_round_fraction_to_f32_bruteforce():
    rng = np.random.default_rng(7)
    cases = [Fraction(1, 3), Fraction(2688), Fraction(1, 2688),
             Fraction(448 * 6) / 7, Fraction(2) ** -149, Fraction(3) * Fraction(2) ** -150]
    for _ in range(300):
        num = int(rng.integers(1, 2 ** 40))
        den = int(rng.integers(1, 2 ** 40))
        cases.append(Fraction(num, den) * Fraction(2) ** int(rng.integers(-60, 60)))
    # exact midpoints between neighbouring fp32 values: ties to even
    for b in [0x3F800000, 0x3F800001, 0x00000001, 0x00000002, 0x4B000001]:
        lo = np.array(b, dtype=np.uint32).view(np.float32)
        hi = np.nextafter(lo, np.float32(np.inf))
        cases.append((Fraction(float(lo)) + Fraction(float(hi))) / 2)
    for q in cases:
        got = formats.round_fraction_to_f32(q)
        exp = _brute_f32(q)
        assert got == exp and np.signbit(got) == np.signbit(exp), q


def _brute_index(v, grid):
    v = Fraction(float(v))
    best = None
    for i, g in enumerate(grid):
        d = abs(Fraction(float(g)) - v)
        key = (d, i % 2)              # nearest, then the even index
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def test_rne_index_on_grid_bruteforce():
    grid = formats.E4M3_VALUES * 3.0
    mids = (grid[:-1] + grid[1:]) / 2
    vals = list(grid) + list(mids)
    vals += [np.nextafter(m, 0) for m in mids] + [np.nextafter(m, np.inf) for m in mids]
    vals += [0.0, 1e-30, 448 * 3.0, 449 * 3.0, 1e30]
    got = formats.rne_index_on_grid(np.array(vals), grid)
    for v, g in zip(vals, got):
        assert g == _brute_index(v, grid), v
