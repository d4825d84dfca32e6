"""Pins for oracle.mxfp4: the scale exponent's closed form, exact round
trip of values on the grid, brute-force nearest-even rounding over every
bf16 magnitude in a fixed block context, and the NVFP4-layout form giving
the same dequantized weight."""
import numpy as np
import pytest

from oracle import formats, mxfp4, nvfp4
from workloads import bf16_from_f32, weight_bf16


def bits(v):
    return bf16_from_f32(np.asarray(v, dtype=np.float32))


def test_scale_exponent_closed_form():
    # floor(log2 amax) - 2: amax 6 -> 2^0, 1 -> 2^-2, 7.9 -> 2^0, 0.3 -> 2^-4
    for amax, e in ((6.0, 0), (1.0, -2), (7.9, 0), (0.3, -4), (1e30, 97), (2.0 ** -120, -122)):
        row = np.zeros((1, 32))
        row[0, 5] = amax
        assert int(mxfp4.scale_bytes(formats.bf16_bits_to_f64(bits(row)))[0, 0]) - 127 == e
    assert mxfp4.scale_bytes(np.zeros((1, 32)))[0, 0] == 0


def test_grid_values_round_trip():
    rng = np.random.default_rng(3)
    e = rng.integers(-20, 20, size=(4, 2))
    c = rng.integers(0, 8, size=(4, 64))
    c[:, 0] = 7
    c[:, 32] = 7                                   # every block's max is 6 X
    sign = rng.integers(0, 2, size=(4, 64))
    vals = np.array(formats.E2M1_MAGNITUDES)[c] * np.ldexp(1.0, np.repeat(e, 32, axis=1))
    vals = np.where(sign == 1, -vals, vals)
    w = bits(vals)
    packed, sb, bad = mxfp4.quantize(w)
    assert not bad
    assert np.array_equal(sb.astype(np.int64) - 127, e)
    assert np.array_equal(mxfp4.dequantize(packed, sb), formats.bf16_bits_to_f64(w))


def test_every_bf16_magnitude_rounds_to_the_nearest_even():
    # block max fixed at 6 (X = 1); the other element sweeps all positive bf16
    # values below 8 and is compared with brute-force nearest (ties to even)
    mags = np.arange(0, 0x4100, dtype=np.uint16)      # 0 .. 7.97 (saturating above 6)
    vals = formats.bf16_bits_to_f64(mags)
    rows = np.zeros((len(mags), 32), dtype=np.uint16)
    rows[:, 0] = bits(6.0)
    rows[:, 1] = mags
    packed, sb, _ = mxfp4.quantize(rows)
    assert np.all(sb == 127)
    got = (packed[:, 0] >> 4) & 7
    grid = np.array(formats.E2M1_MAGNITUDES)
    d = np.abs(vals[:, None] - grid[None, :])
    best = d.min(axis=1)
    for i in range(len(vals)):
        cand = np.nonzero(d[i] == best[i])[0]
        want = cand[0] if len(cand) == 1 else cand[cand % 2 == 0][0]
        assert got[i] == want, (vals[i], got[i], want)


def test_nvfp4_layout_carries_the_same_weight():
    w = weight_bf16(48, 256, 0.02, seed=5, outlier_frac=0.01)
    packed, sb, _ = mxfp4.quantize(w)
    scales, S, ok = mxfp4.to_nvfp4_scales(packed, sb)
    assert ok
    assert np.array_equal(nvfp4.dequantize(packed, scales, S), mxfp4.dequantize(packed, sb))


def test_nvfp4_layout_range_limit():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0
    w[0, 40] = 2.0 ** -30                           # 30 octaves below: out of range
    packed, sb, _ = mxfp4.quantize(bits(w))
    assert not mxfp4.to_nvfp4_scales(packed, sb)[2]
    w[0, 40] = 2.0 ** -15                           # within 17 octaves
    packed, sb, _ = mxfp4.quantize(bits(w))
    scales, S, ok = mxfp4.to_nvfp4_scales(packed, sb)
    assert ok and np.array_equal(nvfp4.dequantize(packed, scales, S), mxfp4.dequantize(packed, sb))
