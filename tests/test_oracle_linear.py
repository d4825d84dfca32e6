"""Pins for oracle.linear: exact rational brute force on tiny inputs and
the identities the pages state (Eq. 2 distributivity, Eq. 9-12 noise
merging, zero-noise / zero-LoRA reductions)."""
from fractions import Fraction

import numpy as np
import pytest

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


# ---- backward through the frozen NVFP4 weight: the layer is linear in x,
# in A and in B separately, so each gradient must satisfy the adjoint
# identity <dy, f(direction)> = <gradient, direction> against the forward
# oracle (a different formula from the one the backward evaluates).

def test_backward_adjoint_identities():
    from workloads import bf16_from_f32
    L = make_layer(m=6, n=40, k=64, r=4, seed=31)
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    z = aqn.sample(31, 0, 0, 0.05, 64)
    rng = np.random.default_rng(31)
    dy = rng.standard_normal((6, 40))
    dx, da, db = linear.backward(dy, L.x, w_hat, z, L.a, L.b, 2.0)
    # x direction: y(v) for a bf16 direction v (y is linear in x)
    v = bf16_from_f32(rng.standard_normal((6, 64)).astype(np.float32))
    yv = linear.linear(v, w_hat, z, L.a, L.b, 2.0)
    assert np.sum(dy * yv) == pytest.approx(np.sum(dx * formats.bf16_bits_to_f64(v)), rel=1e-12)
    # A direction: y(A + V) - y(A) = s x_t V^T B^T
    V = bf16_from_f32(0.02 * rng.standard_normal((4, 64)).astype(np.float32))
    zero_a = np.zeros_like(L.a)
    dyA = linear.linear(L.x, np.zeros_like(w_hat), z, V, L.b, 2.0) - \
        linear.linear(L.x, np.zeros_like(w_hat), z, zero_a, L.b, 2.0)
    assert np.sum(dy * dyA) == pytest.approx(np.sum(da * formats.bf16_bits_to_f64(V)), rel=1e-12)
    # B direction
    U = bf16_from_f32(0.01 * rng.standard_normal((40, 4)).astype(np.float32))
    dyB = linear.linear(L.x, np.zeros_like(w_hat), z, L.a, U, 2.0)
    assert np.sum(dy * dyB) == pytest.approx(np.sum(db * formats.bf16_bits_to_f64(U)), rel=1e-12)


def test_backward_without_lora_or_noise_is_the_transposed_product():
    L = make_layer(m=3, n=24, k=32, r=0, seed=32)
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    dy = np.random.default_rng(32).standard_normal((3, 24))
    dx, da, db = linear.backward(dy, L.x, w_hat)
    assert da is None and db is None
    assert np.array_equal(dx, dy @ w_hat)
