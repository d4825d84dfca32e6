"""Pins for oracle.swiglu: SiLU's closed forms and symmetry, and the split
of the fused gate/up output into its gate and up halves."""
import math

import numpy as np

from oracle import formats, swiglu
from workloads import bf16_from_f32, normal_bf16


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4
    l3 = math.log(3.0)
    np.testing.assert_allclose(swiglu.silu([0.0, l3, -l3]), [0.0, 0.75 * l3, -0.25 * l3],
                               rtol=1e-15, atol=0)
    # sigmoid(g) -> 1 and 0 in the tails; -1000 overflows exp and gives the limit -0
    np.testing.assert_allclose(swiglu.silu([40.0, -40.0]), [40.0, -40.0 * math.exp(-40.0)],
                               rtol=1e-12)
    assert swiglu.silu([-1000.0])[0] == 0.0


def test_silu_symmetry():
    # silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1)
    g = np.linspace(-12.0, 12.0, 241)
    np.testing.assert_allclose(swiglu.silu(g) - swiglu.silu(-g), g, rtol=1e-13, atol=1e-14)


def test_halves_of_the_fused_output():
    m, d = 3, 40
    gate = normal_bf16((m, d), 1.0, 61)
    up = normal_bf16((m, d), 1.0, 62)
    out = swiglu.swiglu(np.hstack([gate, up]))
    g, u = formats.bf16_bits_to_f64(gate), formats.bf16_bits_to_f64(up)
    np.testing.assert_allclose(out, g / (1 + np.exp(-g)) * u, rtol=1e-15)
    # up == 1 leaves SiLU(gate); gate == 0 gives zeros
    ones = bf16_from_f32(np.ones((m, d), dtype=np.float32))
    np.testing.assert_allclose(swiglu.swiglu(np.hstack([gate, ones])), swiglu.silu(g), rtol=1e-15)
    zeros = np.zeros((m, d), dtype=np.uint16)
    assert not swiglu.swiglu(np.hstack([zeros, up])).any()
