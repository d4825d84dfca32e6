"""NVFP4 weight quantizer and dequantizer (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages define NVFP4 by its dequantization [QeRL summary, §3.4, Eq. 6]:
    W_hat = S_FP32 * (S_E4M3 (.) W_tilde)
with one FP32 per-tensor scale, one E4M3 scale per block of 16 contiguous
weights and E2M1 codes W_tilde.  They do not print the quantizer.  The
steps below are the plainest reading that the rest of the pages support:

1. amax = max |W| over the tensor (non-finite input is an error).
2. S = RN_fp32(amax / (6 * 448)): the global scale "ensures the 4-bit values
   fall within the representable range" [QeRL summary, §3.4, text after
   Eq. 6]; 6 is E2M1's largest value [§3.4, E2M1] and 448 is E4M3's.  This
   follows the "scale = range / q_max" rule of Eq. 1 [§3.4, Eq. 1].
3. Per block b of 16 contiguous elements along a row:
   s_b = RNE_E4M3(amax_b / (6 * S)), saturating at 448 (Eq. 1's rule again,
   with q_max = 6, applied on top of S).
4. Per element: code = sign | RNE_E2M1(|w| / (s_b * S)), saturating at 6,
   ties to the even code.  A zero block scale gives magnitude 0.
5. If S == 0 (all-zero tensor, or amax so small that S underflows) every
   scale is 0 and every code keeps only the sign bit.

The quotients in 3 and 4 are taken exactly: rounding onto a grid is
decided by comparing the dividend against (midpoint * divisor), and those
products are exact in fp64 (at most 31 significant bits).  The per-tensor
scale is rounded from an exact rational.

Storage (a reading; the pages fix only "16 contiguous elements"):
  codes  uint8 [N, K/2]   two E2M1 codes per byte, even k in the low nibble
  scales uint8 [N, K/16]  E4M3 bit patterns, block j covers k = 16j..16j+15
  S      float32
where W is the nn.Linear weight [N = out features, K = in features].
"""
from fractions import Fraction

import numpy as np

from .formats import (E2M1_MAGNITUDES, E2M1_MAX, E4M3_MAX, E4M3_VALUES,
                      bf16_bits_to_f64, rne_index_on_grid,
                      round_fraction_to_f32)

BLOCK = 16                     # [QeRL summary, §3.4, Eq. 6]: 16 contiguous
GLOBAL_DIVISOR = E2M1_MAX * E4M3_MAX   # 6 * 448 = 2688

_E2M1 = np.array(E2M1_MAGNITUDES, dtype=np.float64)
_E2M1_MIDS = (_E2M1[:-1] + _E2M1[1:]) * 0.5   # 0.25 0.75 1.25 1.75 2.5 3.5 5


class NonFiniteWeight(ValueError):
    """The weight tensor holds an inf or NaN; NVFP4 has no encoding for it."""


def global_scale(amax):
    """Step 2: S = RN_fp32(amax / 2688), rounded from the exact quotient."""
    return round_fraction_to_f32(Fraction(float(amax)) / int(GLOBAL_DIVISOR))


def block_scale_codes(amax_b, S):
    """Step 3: E4M3 code of RNE(amax_b / (6 S)), saturating at 448.

    amax_b: fp64 array of block maxima.  The grid of E4M3 values is scaled
    by 6*S (exact: S has 24 significant bits), so the rounding decision is
    an exact comparison of amax_b against scaled midpoints.
    """
    S = float(S)
    if S == 0.0:
        return np.zeros(np.shape(amax_b), dtype=np.uint8)
    grid = E4M3_VALUES * (6.0 * S)
    return rne_index_on_grid(amax_b, grid).astype(np.uint8)


def element_magnitude_codes(a, unit):
    """Step 4: RNE_E2M1(a / unit) for a >= 0, ties to even, saturating at 6.

    ``unit`` = s_b * S broadcast against ``a``.  A midpoint t between codes
    i and i+1 is crossed when a > t*unit, or when a == t*unit and i+1 is
    the even code.  t*unit is exact in fp64.  unit == 0 gives code 0.
    """
    a = np.asarray(a, dtype=np.float64)
    unit = np.broadcast_to(np.asarray(unit, dtype=np.float64), a.shape)
    code = np.zeros(a.shape, dtype=np.int64)
    for i, t in enumerate(_E2M1_MIDS):
        thr = t * unit
        if i % 2 == 0:                  # tie stays on code i (even)
            code += a > thr
        else:                           # tie moves up to code i+1 (even)
            code += a >= thr
    code[unit == 0.0] = 0
    return code.astype(np.uint8)


def tensor_amax(w):
    """Step 1: amax = max |w| over the whole tensor (fp64 values)."""
    w = np.asarray(w, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise NonFiniteWeight("non-finite weight")
    return float(np.abs(w).max()) if w.size else 0.0


def encode_with_scale(w, S):
    """Steps 3-5 for rows of a tensor whose global scale S is already known.

    Returns (codes [rows, K/2] uint8, scales [rows, K/16] uint8).  Lets a
    test check sampled rows of a large tensor: S depends on the whole
    tensor, every other step only on the row's own blocks.
    """
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("expected W[N, K] with K a multiple of 16")
    n, k = w.shape
    a = np.abs(w)
    sign = np.signbit(w).astype(np.uint8)
    amax_b = a.reshape(n, k // BLOCK, BLOCK).max(axis=2) if a.size else \
        np.zeros((n, k // BLOCK))
    scodes = block_scale_codes(amax_b, S)
    s_b = E4M3_VALUES[scodes]
    unit = np.repeat(s_b * float(S), BLOCK, axis=1)      # exact products
    mag = element_magnitude_codes(a, unit)
    codes4 = mag | (sign << 3)
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, scodes


def quantize_values(w):
    """Quantize a real-valued [N, K] array (fp64 values) to NVFP4.

    Returns (codes [N, K/2] uint8, scales [N, K/16] uint8, S np.float32).
    Accepts any fp64 input so that the idempotence property
    Q(D(Q(W))) == Q(W) can be checked on dequantized (non-bf16) values.
    """
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("expected W[N, K] with K a multiple of 16")
    S = global_scale(tensor_amax(w))
    packed, scodes = encode_with_scale(w, S)
    return packed, scodes, S


def quantize(w_bits):
    """Quantize a bf16 weight matrix given as uint16 bit patterns [N, K]."""
    return quantize_values(bf16_bits_to_f64(w_bits))


def unpack_codes(packed):
    """uint8 [N, K/2] -> 4-bit codes uint8 [N, K] (even k = low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def e2m1_values(codes4):
    """4-bit codes -> signed E2M1 values (fp64)."""
    codes4 = np.asarray(codes4, dtype=np.uint8)
    mag = _E2M1[codes4 & 7]
    return np.where(codes4 & 8, -mag, mag)


def dequantize(packed, scales, S):
    """Eq. 6 [QeRL summary, §3.4]: W_hat = S_FP32 * (S_E4M3 (.) W_tilde).

    Exact in fp64 (product of a 2-bit, a 4-bit and a 24-bit significand).
    """
    vals = e2m1_values(unpack_codes(packed))
    s_b = np.repeat(E4M3_VALUES[np.asarray(scales, dtype=np.uint8)], BLOCK,
                    axis=1)
    return float(np.float32(S)) * (s_b * vals)

