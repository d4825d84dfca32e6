"""Gated feed-forward activation between the fused gate/up layer and the
down layer (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the feed-forward projections W_gate, W_up and W_down of
the Qwen2.5 models [QeRL summary, §3.4 "Layer coverage"] but not the
function joining them; this follows the Qwen2.5 feed-forward block:
    out[m, j] = SiLU(g[m, j]) * u[m, j],   SiLU(g) = g / (1 + exp(-g))
with g and u the two halves of the fused gate/up output [M, 2 d]: gate in
columns 0 .. d-1, up in columns d .. 2d-1.  Computed in fp64 from the bf16
bit patterns.
"""
import numpy as np

from .formats import bf16_bits_to_f64


def silu(g):
    """g * sigmoid(g) in fp64, written as g / (1 + exp(-g)); exp(-g)
    overflowing to inf for very negative g gives -0 / inf = -0, the limit."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gu_bits):
    """SiLU(gate) * up from the fused gate/up output bits [M, 2 d]."""
    gu = bf16_bits_to_f64(np.atleast_2d(gu_bits))
    d = gu.shape[1] // 2
    return silu(gu[:, :d]) * gu[:, d:]
