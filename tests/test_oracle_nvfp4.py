"""Pins for oracle.nvfp4 against brute force in exact rational arithmetic,
the page-printed format facts, and invariants of the encoding."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, nvfp4
from workloads import bf16_from_f32, weight_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [Fraction(v) for v in formats.E2M1_MAGNITUDES]
E4M3 = [Fraction(float(v)) for v in formats.E4M3_VALUES]


def nearest_even(v, grid):
    """Index of the grid point nearest to v (exact), ties to the even index;
    values above the grid saturate to the top point."""
    best = None
    for i, g in enumerate(grid):
        key = (abs(g - v), i % 2)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def brute_quantize(w_bits):
    """NVFP4 encoding of a tiny bf16 tensor from the definition, in exact
    rationals with exhaustive nearest-point searches (no thresholds)."""
    w = formats.bf16_bits_to_f64(w_bits)
    n, k = w.shape
    amax = max((abs(Fraction(float(v))) for v in w.ravel()), default=Fraction(0))
    S = formats.round_fraction_to_f32(amax / 2688)
    Sq = Fraction(float(S))
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    for i in range(n):
        for b in range(k // 16):
            blk = [Fraction(float(v)) for v in w[i, 16 * b:16 * b + 16]]
            if Sq == 0:
                sc = 0
            else:
                sc = nearest_even(max(abs(v) for v in blk) / (6 * Sq), E4M3)
            scales[i, b] = sc
            unit = E4M3[sc] * Sq
            for j, v in enumerate(blk):
                mag = 0 if unit == 0 else nearest_even(abs(v) / unit, E2M1)
                sign = 1 if np.signbit(w[i, 16 * b + j]) else 0
                codes[i, 16 * b + j] = mag | (sign << 3)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.astype(np.uint8), scales, S


def test_format_facts_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_format.json")))
    assert nvfp4.BLOCK == g["block_size"]
    assert nvfp4.GLOBAL_DIVISOR == 6 * 448


@pytest.mark.parametrize("seed,std,outliers", [(0, 0.02, 0.0), (1, 0.02, 0.05),
                                                (2, 3.0, 0.0), (3, 1e-3, 0.02)])
def test_quantize_matches_bruteforce(seed, std, outliers):
    w = weight_bf16(6, 64, std, seed, outlier_frac=outliers)
    got = nvfp4.quantize(w)
    exp = brute_quantize(w)
    assert np.array_equal(got[0], exp[0])
    assert np.array_equal(got[1], exp[1])
    assert got[2] == exp[2]


def test_quantize_bruteforce_ties_and_specials():
    # blocks built to hit every E2M1 midpoint exactly and every sign of zero
    S_target = 2.0 ** -3
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sb in (1.0, 1.5, 448.0 / 8, 0.875):
        row = [6.0 * sb * S_target]            # anchor: block max -> code 7
        row += [m * sb * S_target for m in mids]
        row += [-m * sb * S_target for m in mids]
        row += [-0.0]
        rows.append(row)
    rows[0][0] = 6.0 * 448.0 * S_target        # tensor max fixes S
    w = bf16_from_f32(np.array(rows, dtype=np.float32))
    got = nvfp4.quantize(w)
    exp = brute_quantize(w)
    assert got[2] == np.float32(S_target)
    assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1])


def exhaustive_bf16_magnitudes():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)      # every finite +bf16
    return bits, formats.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("sb_code,S", [(0x38, 1.0), (0x3D, 2.0 ** -10),
                                       (0x05, 2.0 ** -20 * 1.2345678),
                                       (0x7E, 3.1e-7)])
def test_element_encoder_exhaustive_bf16(sb_code, S):
    """All 32640 finite non-negative bf16 values at a fixed scale context,
    against exhaustive nearest search in exact rationals."""
    S = float(np.float32(S))
    sb = formats.E4M3_VALUES[sb_code]
    bits, a = exhaustive_bf16_magnitudes()
    got = nvfp4.element_magnitude_codes(a, sb * S)
    unit = Fraction(float(sb)) * Fraction(S)
    # brute force by bisection-free scan: classify each value exactly
    vals = [Fraction(float(x)) / unit for x in a]
    exp = [nearest_even(v, E2M1) for v in vals]
    assert np.array_equal(got, np.array(exp, dtype=np.uint8))


def test_block_scale_all_e4m3_midpoints():
    S = float(np.float32(0.37))
    D = Fraction(6) * Fraction(S)
    grid = formats.E4M3_VALUES
    pts = list(grid) + list((grid[:-1] + grid[1:]) / 2)
    amax_b = []
    for p in pts:
        t = float(Fraction(float(p)) * D)     # exact: <= 31 significant bits
        amax_b += [t, np.nextafter(t, 0.0), np.nextafter(t, np.inf)]
    amax_b += [float(500 * D), float(1e-6 * D), 0.0]
    got = nvfp4.block_scale_codes(np.array(amax_b), np.float32(S))
    for v, g in zip(amax_b, got):
        assert g == nearest_even(Fraction(v) / D, E4M3), v


def _grid_tensor(rng, n, k, S):
    """W whose every element is c * s_b * S with each block's max code 7 and
    one block at s_b = 448: exactly representable NVFP4 content."""
    nb = k // 16
    sc = rng.integers(0x08, 0x7F, size=(n, nb))             # normal scales
    sc[0, 0] = 0x7E
    mag = rng.integers(0, 8, size=(n, k))
    mag[:, ::16] = 7
    sign = rng.integers(0, 2, size=(n, k))
    vals = np.array(formats.E2M1_MAGNITUDES)[mag] * np.where(sign, -1.0, 1.0)
    w = vals * np.repeat(formats.E4M3_VALUES[sc], 16, axis=1) * S
    return w, mag | (sign << 3), sc


def test_round_trip_exact_grid_values():
    rng = np.random.default_rng(11)
    S = 2.0 ** -12
    w, codes4, sc = _grid_tensor(rng, 8, 128, S)
    bits = bf16_from_f32(w.astype(np.float32))
    assert np.array_equal(formats.bf16_bits_to_f64(bits), w)   # bf16 exact
    packed, scales, S_got = nvfp4.quantize(bits)
    assert S_got == np.float32(S)
    assert np.array_equal(scales, sc)
    assert np.array_equal(nvfp4.unpack_codes(packed), codes4)
    assert np.array_equal(nvfp4.dequantize(packed, scales, S_got), w)


def test_idempotent_when_block_scales_are_normal():
    w = formats.bf16_bits_to_f64(weight_bf16(16, 256, 0.02, 5, outlier_frac=0.01))
    q1 = nvfp4.quantize_values(w)
    assert np.all(q1[1] >= 0x08)          # generator keeps scales normal
    q2 = nvfp4.quantize_values(nvfp4.dequantize(*q1))
    assert np.array_equal(q1[0], q2[0]) and np.array_equal(q1[1], q2[1])
    assert q1[2] == q2[2]


def test_error_bound():
    """Non-saturated elements lie within half a grid gap of w."""
    w_bits = weight_bf16(32, 512, 0.02, 9, outlier_frac=0.002)
    w = formats.bf16_bits_to_f64(w_bits)
    packed, scales, S = nvfp4.quantize(w_bits)
    w_hat = nvfp4.dequantize(packed, scales, S)
    mag = nvfp4.unpack_codes(packed) & 7
    unit = np.repeat(formats.E4M3_VALUES[scales], 16, axis=1) * float(S)
    gaps = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])  # gap above code
    gaps_below = np.array([0.5, 0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0])
    half = 0.5 * np.maximum(gaps[mag], gaps_below[mag]) * unit
    not_sat = np.abs(w) <= 6.0 * unit
    err = np.abs(w - w_hat)
    assert np.all(err[not_sat] <= half[not_sat])
    # Eq. 5: the static quantization error is W_hat - W, small and nonzero
    assert 0 < np.sqrt(np.mean((w_hat - w) ** 2)) < 0.2 * np.sqrt(np.mean(w ** 2))


def test_zero_tensor_and_signed_zero():
    w = np.zeros((2, 32), dtype=np.uint16)
    w[1, 3] = 0x8000                       # -0.0
    packed, scales, S = nvfp4.quantize(w)
    assert S == 0 and not np.any(scales)
    codes = nvfp4.unpack_codes(packed)
    assert codes[1, 3] == 8 and np.count_nonzero(codes) == 1
    assert np.all(nvfp4.dequantize(packed, scales, S) == 0)


def test_underflowing_block_scale_gives_zero_block():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 1.0            # tensor max
    w[0, 16] = 1e-7          # amax_b / (6 S) far below 2**-10
    w[0, 17] = -1e-7
    packed, scales, S = nvfp4.quantize(bf16_from_f32(w))
    assert scales[0, 1] == 0
    codes = nvfp4.unpack_codes(packed)
    assert codes[0, 16] == 0 and codes[0, 17] == 8


def test_nonfinite_and_shape_errors():
    w = np.zeros((1, 16), dtype=np.uint16)
    w[0, 5] = 0x7F80                      # +inf
    with pytest.raises(nvfp4.NonFiniteWeight):
        nvfp4.quantize(w)
    w[0, 5] = 0x7FC1                      # NaN
    with pytest.raises(nvfp4.NonFiniteWeight):
        nvfp4.quantize(w)
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((2, 24), dtype=np.uint16))


def test_dequantize_eq6_hand_example():
    # codes: +6, -0.5, +1.5, -4 ; block scale 1.25 (E4M3 0x3A), S = 0.5
    codes = np.array([[0x7, 0x9, 0x3, 0xE] + [0] * 12], dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.array([[0x3A]], dtype=np.uint8)
    assert formats.E4M3_VALUES[0x3A] == 1.25
    w_hat = nvfp4.dequantize(packed, scales, np.float32(0.5))
    assert list(w_hat[0, :4]) == [3.75, -0.3125, 0.9375, -2.5]
    assert not np.any(w_hat[0, 4:])


def test_global_scale_is_rounded_quotient():
    for amax in [1.0, 0.4, 3.0e38, 1e-40, 0.0, 2688.0, 6.0 * 448 * 2.0 ** -140]:
        S = nvfp4.global_scale(amax)
        assert S == np.float32(np.float64(amax) / 2688.0)
