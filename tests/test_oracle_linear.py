"""Pins for oracle.linear: exact rational brute force on tiny inputs and
the identities the pages state (Eq. 2 distributivity, Eq. 9-12 noise
merging, zero-noise / zero-LoRA reductions)."""
from fractions import Fraction

import numpy as np

from oracle import aqn, formats, linear, nvfp4
from workloads import make_layer


def _frac(v):
    return Fraction(float(v))


def test_linear_matches_exact_rationals():
    L = make_layer(m=2, n=3, k=32, r=2, seed=4)
    q = nvfp4.quantize(L.w)
    w_hat = nvfp4.dequantize(*q)
    z = aqn.sample(4, 0, 0, 0.05, 32)
    y = linear.linear(L.x, w_hat, z, L.a, L.b, 2.0)
    x = formats.bf16_bits_to_f64(L.x)
    a = formats.bf16_bits_to_f64(L.a)
    b = formats.bf16_bits_to_f64(L.b)
    for mi in range(2):
        xt = [_frac(x[mi, k]) * (1 + _frac(z[k])) for k in range(32)]
        t = [sum(xt[k] * _frac(a[j, k]) for k in range(32)) for j in range(2)]
        for ni in range(3):
            exact = sum(xt[k] * _frac(w_hat[ni, k]) for k in range(32))
            exact += 2 * sum(t[j] * _frac(b[ni, j]) for j in range(2))
            assert abs(_frac(y[mi, ni]) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)


def test_zero_noise_and_zero_lora_reduce_to_plain_matmul():
    L = make_layer(m=5, n=48, k=64, r=4, seed=5)
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    x = formats.bf16_bits_to_f64(L.x)
    plain = x @ w_hat.T
    assert np.array_equal(linear.linear(L.x, w_hat), plain)
    z0 = np.zeros(64, dtype=np.float32)
    assert np.array_equal(linear.linear(L.x, w_hat, z0), plain)
    b0 = np.zeros_like(L.b)
    assert np.array_equal(linear.linear(L.x, w_hat, None, L.a, b0, 2.0), plain)


def test_noise_merge_identity_eq12():
    """x (.) (1+z) times W_hat^T == x times (W_hat with column j scaled by
    1 + z_j)^T (the multiplicative form of Eq. 11-12 with w == 1)."""
    L = make_layer(m=7, n=40, k=96, r=0, seed=6)
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    z = aqn.sample(6, 0, 3, 0.01, 96)
    lhs = linear.linear(L.x, w_hat, z)
    rhs = formats.bf16_bits_to_f64(L.x) @ (w_hat * (1.0 + z.astype(np.float64))).T
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-14)


def test_lora_distributivity_eq2():
    """x_t (W_hat + s B A)^T == x_t W_hat^T + s (x_t A^T) B^T."""
    L = make_layer(m=3, n=32, k=64, r=8, seed=7)
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    z = aqn.sample(7, 0, 0, 0.01, 64)
    a = formats.bf16_bits_to_f64(L.a)
    b = formats.bf16_bits_to_f64(L.b)
    merged = w_hat + 2.0 * (b @ a)
    lhs = linear.noisy_input(L.x, z) @ merged.T
    rhs = linear.linear(L.x, w_hat, z, L.a, L.b, 2.0)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-13)
    t = linear.lora_down(L.x, z, L.a)
    assert np.allclose(linear.noisy_input(L.x, z) @ w_hat.T + 2.0 * t @ b.T, rhs,
                       rtol=1e-12, atol=1e-13)


def test_max_rel_error_metric():
    y_ref = np.array([1.0, -2.0, 0.0, 1e-9])
    assert linear.max_rel_error(y_ref, y_ref) == 0.0
    rms = np.sqrt(np.mean(y_ref ** 2))
    y = y_ref.copy()
    y[2] = 0.01
    assert linear.max_rel_error(y, y_ref) == 0.01 / rms
