"""MXFP4: E2M1 codes with one power-of-two (E8M0) scale per 32 elements
(oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages describe MXFP4 as E2M1 elements sharing an E8M0 scale over
blocks of 32 [QeRL summary, §3.4, the format list beside NVFP4]; the scale
rule is not on the pages and follows the OCP Microscaling (MX) v1.0
specification:
    X    = 2^(floor(log2(amax_b)) - 2)       2 = exponent of E2M1's largest value 6
    byte = floor(log2(amax_b)) - 2 + 127, clamped to [0, 254]; amax_b = 0 -> 0
    code = sign | RNE_E2M1,sat(|w| / X)      ties to even, saturating at 6
    W_hat = X * e2m1(code)
|w| / X is a power-of-two scaling of a bf16 value, so every step is exact
in fp64.  Codes pack two per byte with the even k in the low nibble, as
for NVFP4.

to_nvfp4_scales re-expresses the scales in this library's NVFP4 layout
(one E4M3 per 16 elements and an FP32 tensor scale) so that the NVFP4
kernels compute the MXFP4 layer exactly: S = 2^(E_max - 8) and each block
scale 2^(e - E_max + 8), an E4M3 power of two as long as e >= E_max - 17.
"""
import numpy as np

from .formats import E2M1_MAGNITUDES, bf16_bits_to_f64, rne_index_on_grid
from .nvfp4 import e2m1_values, unpack_codes

BLOCK = 32


def scale_bytes(w):
    """E8M0 scale byte per 32-element block of w [N, K] (fp64 values)."""
    n, k = w.shape
    amax = np.max(np.abs(w.reshape(n, k // BLOCK, BLOCK)), axis=2)
    _, ex = np.frexp(amax)                       # amax = f 2^ex, f in [0.5, 1)
    byte = np.clip(ex - 1 - 2 + 127, 0, 254)
    return np.where(amax > 0, byte, 0).astype(np.uint8)


def quantize(w_bits):
    """bf16 bits [N, K] -> (codes uint8 [N, K/2], scales uint8 [N, K/32],
    nonfinite).  K % 32 == 0."""
    w = bf16_bits_to_f64(np.asarray(w_bits))
    if not np.all(np.isfinite(w)):
        return None, None, True
    n, k = w.shape
    sb = scale_bytes(w)
    x = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), BLOCK, axis=1)
    mag = rne_index_on_grid(np.abs(w) / x, E2M1_MAGNITUDES).astype(np.uint8)
    sign = (np.asarray(w_bits, dtype=np.uint16) >> 15).astype(np.uint8)
    c = mag | (sign << 3)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb, False


def dequantize(packed, sbytes):
    """W_hat = 2^(byte - 127) * e2m1(code), fp64 [N, K]."""
    vals = e2m1_values(unpack_codes(packed))
    x = np.repeat(np.ldexp(1.0, np.asarray(sbytes, dtype=np.int64) - 127), BLOCK, axis=1)
    return x * vals


def to_nvfp4_scales(packed, sbytes):
    """(E4M3 scale codes [N, K/16], S, ok): the same weight in the NVFP4
    layout.  ok is False when a block with a nonzero code has its exponent
    more than 17 below the largest (no E4M3 power of two can carry it)."""
    sb = np.asarray(sbytes, dtype=np.int64)
    emax = int(sb.max()) - 127
    big_e = emax - 8
    rel = sb - 127 - big_e                          # block exponent relative to S, <= 8
    nz = (unpack_codes(packed) & 7).reshape(sb.shape[0], sb.shape[1], BLOCK).any(axis=2)
    ok = not np.any(nz & (rel < -9))
    # E4M3 code of 2^j: normal (j + 7) << 3 for j >= -6, subnormal 2^(j + 9) below
    code = np.where(rel >= -6, (rel + 7) << 3, np.left_shift(1, np.clip(rel + 9, 0, 2)))
    code = np.where(rel < -9, 0, code).astype(np.uint8)
    return np.repeat(code, 2, axis=1), float(np.ldexp(np.float32(1.0), big_e)), ok
