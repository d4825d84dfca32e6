"""Adaptive Quantization Noise: sigma schedule and noise vector (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Schedule [QeRL summary, §3.4 "The exponential decay schedule", Eq. 8]:
    sigma(k) = sigma_start * (sigma_end / sigma_start) ** ((k - 1) / (K - 1))
for stages k = 1..K, with sigma(0) = 0: stage 0 carries only the
quantization noise [§3.4 "Stage 0: pure quantization noise"].  The paper's
values are sigma_start = 1e-2, sigma_end = 5e-4, K = 10 [§3.4, Table 4
hyperparameters].  K == 1 has a single stage at sigma_start (the formula
divides by K - 1; this is the only reading that keeps sigma(1) ==
sigma_start).

Noise [QeRL summary, §3.4 "The stochastic noise vector", Eq. 7]:
Z_noisy ~ N(0, sigma^2 I), a vector of length d = the layer's input
dimension, drawn afresh for every forward pass.  The pages do not say how
the normal numbers are produced.  The oracle and the HIP library both use
  * Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and
    Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), with
      key     = (seed, stream_id)
      counter = (j // 4, call_id, row, 0) for noise element j, row = 0 for
                the vector shared by a call's token rows, row = i for token
                row i when every rollout draws its own;
  * the Box-Muller transform (Box and Muller, 1958) on the four 64-bit
    output words (r0, r1, r2, r3) of that counter:
      u1 = ((r >> 11) + 1) * 2**-53  in (0, 1]   from r0 (resp. r2)
      u2 =  (r >> 11)      * 2**-53  in [0, 1)   from r1 (resp. r3)
      rad = sqrt(-2 ln u1)
      n_{4q+0} = rad(r0) cos(2 pi u2(r1)),  n_{4q+1} = rad(r0) sin(2 pi u2(r1))
      n_{4q+2} = rad(r2) cos(2 pi u2(r3)),  n_{4q+3} = rad(r2) sin(2 pi u2(r3))
    all in fp64;
  * z_j = RN_fp32(sigma * n_j).
"""
import math

import numpy as np

MASK64 = (1 << 64) - 1
# Philox4x64 constants (Salmon et al. 2011): multipliers and Weyl key bumps.
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
PHILOX_ROUNDS = 10


def sigma(sigma_start, sigma_end, num_stages, stage):
    """Eq. 8 with sigma(0) = 0 [QeRL summary, §3.4]."""
    sigma_start, sigma_end = float(sigma_start), float(sigma_end)
    num_stages, stage = int(num_stages), int(stage)
    if num_stages < 1 or not 0 <= stage <= num_stages:
        raise ValueError("need K >= 1 and 0 <= k <= K")
    if not (sigma_start > 0 and sigma_end > 0):
        raise ValueError("sigma_start and sigma_end must be positive")
    if stage == 0:
        return 0.0
    if num_stages == 1:
        return sigma_start
    ratio = sigma_end / sigma_start
    return sigma_start * ratio ** ((stage - 1) / (num_stages - 1))


SCHEDULES = ("exponential", "linear", "cosine", "logarithmic")


def sigma_schedule(mode, sigma_start, sigma_end, num_stages, stage):
    """sigma at stage k under one of the four decay schedules the pages
    compare [QeRL summary, §3.4, "Why exponential decay" (Fig. 9, Fig. 15)];
    with t = (k - 1) / (K - 1):
      exponential  sigma_start (sigma_end / sigma_start)^t          (Eq. 8)
      linear       sigma_start - (sigma_start - sigma_end) t
      cosine       sigma_end + (sigma_start - sigma_end) (1 + cos(pi t)) / 2
      logarithmic  sigma_start - (sigma_start - sigma_end) log(k) / log(K)
    sigma(0) = 0 and K = 1 gives sigma_start, as for Eq. 8."""
    if mode not in SCHEDULES:
        raise ValueError(f"unknown schedule {mode!r}")
    if mode == "exponential":
        return sigma(sigma_start, sigma_end, num_stages, stage)
    sigma_start, sigma_end = float(sigma_start), float(sigma_end)
    num_stages, stage = int(num_stages), int(stage)
    if num_stages < 1 or not 0 <= stage <= num_stages:
        raise ValueError("need K >= 1 and 0 <= k <= K")
    if not (sigma_start > 0 and sigma_end > 0):
        raise ValueError("sigma_start and sigma_end must be positive")
    if stage == 0:
        return 0.0
    if num_stages == 1:
        return sigma_start
    t = (stage - 1) / (num_stages - 1)
    span = sigma_start - sigma_end
    if mode == "linear":
        return sigma_start - span * t
    if mode == "cosine":
        return sigma_end + 0.5 * span * (1.0 + math.cos(math.pi * t))
    return sigma_start - span * math.log(stage) / math.log(num_stages)


def _mulhilo(a, b):
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64(counter, key, rounds=PHILOX_ROUNDS):
    """One Philox4x64 block: 4 x 64-bit counter, 2 x 64-bit key -> 4 words.

    Each round multiplies counter words 0 and 2 by the two constants,
    crosses the halves and xors in the key; the key is bumped by the two
    Weyl constants between rounds.  Pure Python integers, one block at a
    time (slow and plain on purpose).
    """
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for rnd in range(rounds):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def box_muller_pair(r_a, r_b):
    """Two standard normals from two 64-bit words (fp64 Box-Muller)."""
    u1 = ((int(r_a) >> 11) + 1) * 2.0 ** -53
    u2 = (int(r_b) >> 11) * 2.0 ** -53
    rad = math.sqrt(-2.0 * math.log(u1))
    ang = 2.0 * math.pi * u2
    return rad * math.cos(ang), rad * math.sin(ang)


def standard_normals(seed, stream_id, call_id, d, row=0):
    """n_0..n_{d-1} for (seed, stream_id, call_id), fp64; `row` is counter
    word 2 (0 for the noise vector shared by the rows of a call, i for
    token row i of the per-rollout variant)."""
    out = np.empty(int(d), dtype=np.float64)
    for q in range((int(d) + 3) // 4):
        r0, r1, r2, r3 = philox4x64((q, call_id, row, 0), (seed, stream_id))
        vals = box_muller_pair(r0, r1) + box_muller_pair(r2, r3)
        for i in range(4):
            j = 4 * q + i
            if j < d:
                out[j] = vals[i]
    return out


def sample(seed, stream_id, call_id, sig, d, row=0):
    """AQN noise vector z (fp32 [d]) [QeRL summary, §3.4, Eq. 7]."""
    n = standard_normals(seed, stream_id, call_id, d, row)
    return (float(sig) * n).astype(np.float32)


def sample_rows(seed, stream_id, call_id, sig, m, d):
    """One noise vector per token row (fp32 [m, d]): the variant in which
    every rollout of a batch sees its own draw [QeRL summary, §3.4 "Noise
    injection frequency"].  Row i uses counter word 2 = i, so row 0 is the
    shared vector of `sample`."""
    return np.stack([sample(seed, stream_id, call_id, sig, d, row=i) for i in range(int(m))])
