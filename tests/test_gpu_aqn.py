"""GPU noise parity: z from qerl_aqn_sample against the oracle's Philox4x64
+ Box-Muller, within one fp32 ulp (fp64 libm and the device math library
may differ in the last fp64 bit), plus statistics and the counter
properties."""
import math

import numpy as np
import pytest
import torch

from oracle import aqn
from tests._gpu import host

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402


def gpu_z(seed, stream, call, sigma, d):
    z = q.qerl_aqn_sample(seed, stream, call, sigma, d, device="cuda:0")
    torch.cuda.synchronize()
    return host(z)


def ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("seed,stream,call,stage,d", [
    (0, 0, 0, 3, 256), (1, 2, 3, 1, 3584), (2 ** 63 + 5, 7, 2 ** 40, 10, 27648),
    (42, 0, 1, 5, 1), (42, 0, 1, 5, 5), (9, 1, 0, 1, 18944)])
def test_noise_matches_oracle(seed, stream, call, stage, d):
    sig = aqn.sigma(1e-2, 5e-4, 10, stage)
    assert q.qerl_aqn_sigma(1e-2, 5e-4, 10, stage) == pytest.approx(sig, rel=1e-15)
    z = gpu_z(seed, stream, call, sig, d)
    ref = aqn.sample(seed, stream, call, sig, d)
    diff = ulp_diff(z, ref)
    assert diff.max() <= 1
    assert np.mean(diff == 0) >= 0.99


def test_zero_sigma_and_prefix():
    assert not np.any(gpu_z(3, 0, 0, 0.0, 1000))
    full = gpu_z(5, 1, 2, 0.01, 4096)
    assert np.array_equal(gpu_z(5, 1, 2, 0.01, 13), full[:13])
    assert not np.array_equal(gpu_z(5, 1, 3, 0.01, 4096), full)


def test_noise_statistics_large():
    d = 1 << 22
    sig = 0.01
    z = gpu_z(77, 0, 0, sig, d).astype(np.float64) / sig
    assert abs(z.mean()) < 5 / math.sqrt(d)
    assert abs(z.std() - 1) < 5 / math.sqrt(2 * d)
    # tail mass beyond 3 sigma: 0.0027 two-sided
    tail = np.mean(np.abs(z) > 3)
    assert abs(tail - 0.0026998) < 5 * math.sqrt(0.0027 / d)


@pytest.mark.parametrize("count,stride,d", [(3, 4, 5120), (64, 4, 27648), (5, 1, 7), (2, 0, 100)])
def test_batch_rows_equal_single_calls(count, stride, d):
    # qerl_aqn_sample_batch: row i is the vector of call id c0 + i * stride,
    # bit for bit, and within one fp32 ulp of the oracle's
    sig, c0 = 0.01, 1000 + stride
    zb = q.qerl_aqn_sample_batch(11, 2, c0, stride, count, sig, d, device="cuda:0")
    torch.cuda.synchronize()
    zb = host(zb)
    assert zb.shape == (count, d)
    for i in sorted({0, count // 2, count - 1}):
        assert np.array_equal(zb[i], gpu_z(11, 2, c0 + i * stride, sig, d))
        assert ulp_diff(zb[i], aqn.sample(11, 2, c0 + i * stride, sig, d)).max() <= 1
