"""Pins for oracle.rmsnorm: exact values where the normalisation is a
perfect square, closed forms (a two-element row, a one-hot row), the
scale invariance and unit RMS of the normalisation, and the two other
forms the pages give for the same noise: the multiplier (1 + z / w) on
the plain RMSNorm output (Eq. 11) and the scaling of the next weight's
input channels (Eq. 12)."""
import numpy as np

from oracle import aqn, formats, rmsnorm
from workloads import bf16_from_f32, norm_inputs


def bits(v):
    return bf16_from_f32(np.asarray(v, dtype=np.float32))


def test_exact_when_mean_square_plus_delta_is_a_square():
    # mean([1, 2, 2]^2) = 3, + delta 1 = 4: the divisor is exactly 2, so
    # y = (w + z) x / 2 exactly; delta added to the sum instead of the
    # mean, or outside the root, gives other values.
    x = bits([[1.0, 2.0, 2.0]])
    w = bits([1.0, 1.0, 1.0])
    z = np.array([0.5, -0.25, 0.0], dtype=np.float32)
    y = rmsnorm.rmsnorm_noisy(x, w, z, delta=1.0)
    assert np.array_equal(y, [[0.75, 0.75, 1.0]])


def test_two_element_closed_form():
    x = bits([[3.0, 4.0], [-3.0, 4.0]])
    w = bits([1.0, 0.5])
    y = rmsnorm.rmsnorm_noisy(x, w, None, delta=0.0)
    r = np.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 0.5 * 4 / r], [-3 / r, 0.5 * 4 / r]], rtol=1e-15)


def test_one_hot_row():
    n, j, a = 16, 5, -2.5
    row = np.zeros(n, dtype=np.float32)
    row[j] = a
    _, w = norm_inputs(1, n, seed=3)
    z = aqn.sample(3, 0, 0, 0.01, n)
    y = rmsnorm.rmsnorm_noisy(bits([row]), w, z, delta=0.0)[0]
    # mean square a^2 / n: the divisor is |a| / 4, so y_j = -4 (w_j + z_j)
    wz = formats.bf16_bits_to_f64(w) + z.astype(np.float64)
    expect = np.zeros(n)
    expect[j] = -4.0 * wz[j]
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)


def test_scale_invariance_and_unit_rms():
    x, w = norm_inputs(6, 96, seed=4)
    ones = bits(np.ones(96))
    y = rmsnorm.rmsnorm_noisy(x, ones, None, delta=0.0)
    # every row has unit RMS, whatever its own scale
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    # a power-of-two scale of x changes nothing at all
    x4 = bits(4.0 * formats.bf16_bits_to_f64(x))
    assert np.array_equal(rmsnorm.rmsnorm_noisy(x4, w, None, delta=0.0),
                          rmsnorm.rmsnorm_noisy(x, w, None, delta=0.0))


def test_rows_are_normalised_independently():
    # Row 1 is row 0 times 8: with delta 0 both rows give the same output,
    # which a mean taken over the wrong axis would not.
    x0, w = norm_inputs(1, 40, seed=5)
    x = np.vstack([x0, bits(8.0 * formats.bf16_bits_to_f64(x0))])
    y = rmsnorm.rmsnorm_noisy(x, w, None, delta=0.0)
    assert np.array_equal(y[0], y[1])


def test_no_noise_equals_zero_noise():
    x, w = norm_inputs(3, 64, seed=6)
    assert np.array_equal(rmsnorm.rmsnorm_noisy(x, w, None),
                          rmsnorm.rmsnorm_noisy(x, w, np.zeros(64, dtype=np.float32)))


def test_eq11_multiplier_on_plain_rmsnorm():
    # (w + z) x / rms == (1 + z / w) (.) (w x / rms)   [§3.4, Eq. 11]
    x, w = norm_inputs(5, 128, seed=7)
    z = aqn.sample(7, 0, 1, 0.01, 128)
    plain = rmsnorm.rmsnorm_noisy(x, w, None)
    wf = formats.bf16_bits_to_f64(w)
    form11 = (1.0 + z.astype(np.float64) / wf) * plain
    np.testing.assert_allclose(rmsnorm.rmsnorm_noisy(x, w, z), form11, rtol=1e-13)


def test_eq12_noise_moves_onto_weight_input_channels():
    # RMSNorm_noise(X) W^T == RMSNorm(X) ((1 + z / w)^T (.) W)^T   [§3.4, Eq. 12]:
    # the noise scales the input channels (columns) of the next weight.
    x, w = norm_inputs(4, 64, seed=8)
    z = aqn.sample(8, 0, 2, 0.01, 64)
    W = np.random.default_rng(8).standard_normal((24, 64))
    wf = formats.bf16_bits_to_f64(w)
    lhs = rmsnorm.rmsnorm_noisy(x, w, z) @ W.T
    rhs = rmsnorm.rmsnorm_noisy(x, w, None) @ ((1.0 + z.astype(np.float64) / wf)[None, :] * W).T
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)
