"""Noisy RMSNorm, the producer of the noisy activations (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition [QeRL summary, §3.4 "Noise Merging", Eq. 10], in fp64:
    y[m, i] = (w_i + z_i) * x[m, i] / sqrt( (1/N) sum_j x[m, j]^2 + delta )
for every token row m of x [M, N]: the AQN noise vector z (length N, one
draw per forward pass, shared by the rows of a call) is added to the
RMSNorm scale w, and the normalisation itself is unchanged.  z None means
no noise (plain RMSNorm).  x and w are bf16 bit patterns, z is fp32.

The pages restate the same operation as a multiplier on the plain RMSNorm
output, (1 + z / w) (.) RMSNorm(x) (Eq. 11), and, pushed through the next
linear layer, as a scaling of the weight's input channels (Eq. 12); the
tests pin this function to both forms.
"""
import numpy as np

from .formats import bf16_bits_to_f64


def rmsnorm_noisy(x_bits, w_bits, z=None, delta=1e-6):
    """(w + z) (.) x / sqrt(mean(x^2) + delta) per row, fp64 [M, N]."""
    x = bf16_bits_to_f64(np.atleast_2d(x_bits))
    w = bf16_bits_to_f64(w_bits)
    scale = w if z is None else w + np.asarray(z, dtype=np.float32).astype(np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return scale * (x / np.sqrt(ms + float(delta)))
