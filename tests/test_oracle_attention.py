"""Pins for oracle.attention and for the per-rollout noise of oracle.aqn and
oracle.linear: closed forms of softmax attention (one position, equal keys,
a dominant key), the grouped-query head map, and the row structure of the
per-row noise."""
import math

import numpy as np

from oracle import aqn, attention, formats, linear
from workloads import bf16_from_f32, make_layer, normal_bf16


def test_single_position_outputs_the_value_of_the_group():
    # softmax over one score is exactly 1: query head h reads v of head h // g
    n_q, n_kv, d, m = 6, 2, 8, 3
    qkv = normal_bf16((m, (n_q + 2 * n_kv) * d), 1.0, 5)
    out = attention.decode_attention(qkv, n_q, n_kv, d)
    vals = formats.bf16_bits_to_f64(qkv)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        v = vals[:, (n_q + n_kv + g) * d:(n_q + n_kv + g + 1) * d]
        assert np.array_equal(out[:, h * d:(h + 1) * d], v)


def test_equal_keys_average_the_values():
    # two context positions with the same key: weights 1/2 each
    n_q, n_kv, d = 2, 1, 4
    qkv = normal_bf16((1, (n_q + 2 * n_kv) * d), 1.0, 6)
    _, k, v = attention.split_qkv(formats.bf16_bits_to_f64(qkv), n_q, n_kv, d)
    past_v = np.full((1, 1, n_kv, d), 3.0)
    out = attention.decode_attention(qkv, n_q, n_kv, d, past_k=k[:, None], past_v=past_v)
    for h in range(n_q):
        assert np.allclose(out[0, h * d:(h + 1) * d], 0.5 * (v[0, 0] + 3.0), atol=1e-15)


def test_dominant_key_selects_its_value():
    n_q, n_kv, d = 1, 1, 4
    q = np.array([40.0, 0, 0, 0])
    qkv = bf16_from_f32(np.concatenate([q, [1.0, 0, 0, 0], [7.0, 7.0, 7.0, 7.0]])[None])
    past_k = np.array([[[[-1.0, 0, 0, 0]]]])
    past_v = np.array([[[[-5.0, -5.0, -5.0, -5.0]]]])
    out = attention.decode_attention(qkv, n_q, n_kv, d, past_k, past_v)
    # weight of the past key: 1 / (1 + e^{(40 - (-40)) / 2})
    w_past = 1.0 / (1.0 + math.exp(40.0))
    assert np.allclose(out[0], 7.0 * (1 - w_past) - 5.0 * w_past, rtol=1e-15)


def test_row_noise_row0_is_the_shared_vector_and_rows_are_independent():
    z = aqn.sample_rows(3, 1, 7, 0.01, 6, 4096)
    assert z.shape == (6, 4096) and z.dtype == np.float32
    assert np.array_equal(z[0], aqn.sample(3, 1, 7, 0.01, 4096))
    # row i is counter word 2 = i of the generator pinned to numpy's Philox
    r = aqn.philox4x64((5, 7, 4, 0), (3, 1))
    n = aqn.box_muller_pair(r[0], r[1]) + aqn.box_muller_pair(r[2], r[3])
    assert np.array_equal(z[4, 20:24], (0.01 * np.array(n)).astype(np.float32))
    for i in range(6):
        for j in range(i + 1, 6):
            assert abs(np.corrcoef(z[i], z[j])[0, 1]) < 5.0 / math.sqrt(4096)


def test_row_noise_layer_is_the_rowwise_layer():
    # with one noise row per token, row i of y is the layer applied to row i
    # of x with that row's noise as the shared vector
    L = make_layer(5, 48, 64, 8, seed=9)
    w = np.random.default_rng(1).standard_normal((48, 64)) * 0.02
    z = aqn.sample_rows(9, 0, 1, 0.25, 5, 64)
    y = linear.linear(L.x, w, z, L.a, L.b, 2.0)
    for i in range(5):
        yi = linear.linear(L.x[i:i + 1], w, z[i], L.a, L.b, 2.0)
        assert np.allclose(y[i], yi[0], rtol=1e-13, atol=1e-15)
    # equal rows reduce to the shared-noise layer
    zs = np.broadcast_to(z[0], (5, 64))
    assert np.allclose(linear.linear(L.x, w, zs, L.a, L.b, 2.0),
                       linear.linear(L.x, w, z[0], L.a, L.b, 2.0), rtol=1e-13, atol=1e-15)
