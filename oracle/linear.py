"""NVFP4 linear layer with LoRA side branch and AQN noise (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition, in fp64 throughout:
    x_t = x (.) (1 + z)                                   (per input channel)
    y   = x_t W_hat^T + s (x_t A^T) B^T
with
  * W_hat [N, K] the NVFP4 dequantized weight (Eq. 6, oracle.nvfp4);
  * LoRA [QeRL summary, §3.4 "Low-Rank Adaptation", Eq. 2]: the effective
    weight is W_hat + B A with B [d x r] and A [r x k]; here A is [r, K],
    B is [N, r] and s = alpha / r scales the branch (the usual LoRA
    scaling; the pages name alpha as "LoRA alpha (scaling factor)" in the
    Algorithm 1 hyperparameters);
  * AQN noise merged into the preceding RMSNorm [QeRL summary, §3.4
    "Noise Merging", Eq. 10-12]: the noise multiplies every input channel
    j of the activations by (1 + z_j / w_j).  With the RMSNorm weight w
    folded into the activations (w == 1 here) this is x_j (1 + z_j), and
    the same noisy activations feed both the quantized path and the LoRA
    path [§3.4, "Interaction with AQN noise"].  One z of length K is shared
    by all M rows of a call (Eq. 9: the noise row vector is broadcast
    across the batch).

numpy's fp64 matmul is used as the textbook routine for the contractions;
nothing is blocked, fused or reordered beyond the definition.
"""
import numpy as np

from .formats import bf16_bits_to_f64


def noisy_input(x_bits, z):
    """x_t = x (.) (1 + z) in fp64; z None means no noise (x_t = x)."""
    x = bf16_bits_to_f64(x_bits)
    if z is None:
        return x
    return x * (1.0 + np.asarray(z, dtype=np.float32).astype(np.float64))


def linear(x_bits, w_hat, z=None, a_bits=None, b_bits=None, lora_scale=0.0):
    """y [M, N] fp64 = x_t W_hat^T + s (x_t A^T) B^T."""
    return linear_values(bf16_bits_to_f64(x_bits), w_hat, z, a_bits, b_bits, lora_scale)


def linear_values(x, w_hat, z=None, a_bits=None, b_bits=None, lora_scale=0.0):
    """The same layer for activations given as fp64 values (a chain of
    layers evaluated without rounding in between)."""
    x = np.asarray(x, dtype=np.float64)
    xt = x if z is None else x * (1.0 + np.asarray(z, dtype=np.float32).astype(np.float64))
    y = xt @ np.asarray(w_hat, dtype=np.float64).T
    if a_bits is not None and b_bits is not None and np.size(a_bits):
        a = bf16_bits_to_f64(a_bits)
        b = bf16_bits_to_f64(b_bits)
        y = y + float(lora_scale) * ((xt @ a.T) @ b.T)
    return y


def lora_down(x_bits, z, a_bits):
    """t = x_t A^T (fp64 [M, r]): the LoRA down projection."""
    return noisy_input(x_bits, z) @ bf16_bits_to_f64(a_bits).T


def max_rel_error(y, y_ref):
    """max_i |y_i - y*_i| / max(|y*_i|, rms(y*)).

    The floor at rms(y*) keeps outputs that cancel to nearly zero from
    dominating an elementwise ratio.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    den = np.maximum(np.abs(y_ref), rms)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(np.abs(y - y_ref) / den))


def backward(dy, x_bits, w_hat, z=None, a_bits=None, b_bits=None, lora_scale=0.0):
    """Gradients of the layer through the frozen NVFP4 weight, fp64.

    The rollout's log-probabilities are taken on the same quantized model
    and only the LoRA factors (and the RMSNorm scales) are trained
    [QeRL summary, §3.4 "Low-Rank Adaptation" and Algorithm 1's inner
    updates]: W_hat gets no gradient, the input does (it flows on to the
    layers below).  With x_t = x (.) (1 + z), t = x_t A^T and g = dy B:
        dx = (dy W_hat + s g A) (.) (1 + z)
        dA = s g^T x_t          dB = s dy^T t
    dy [M, N] fp64 values; returns (dx [M, K], dA [r, K], dB [N, r]) (the
    last two None without a LoRA branch)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = bf16_bits_to_f64(x_bits)
    zz = np.zeros(x.shape[1]) if z is None else np.asarray(z, dtype=np.float32).astype(np.float64)
    xt = x * (1.0 + zz)
    dxt = dy @ np.asarray(w_hat, dtype=np.float64)
    if a_bits is None or b_bits is None or not np.size(a_bits):
        return dxt * (1.0 + zz), None, None
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    s = float(lora_scale)
    g = dy @ b
    dxt = dxt + s * (g @ a)
    return dxt * (1.0 + zz), s * (g.T @ xt), s * (dy.T @ (xt @ a.T))
