"""GPU parity of the noisy RMSNorm producer (qerl_rmsnorm_noisy) against
the fp64 oracle [QeRL summary, §3.4 "Noise Merging", Eq. 10].

Bar: every output is a faithful bf16 rounding of the exact value, i.e.
|y - y*| <= one bf16 ulp of y* (the kernel sums squares and scales in
fp32, so its pre-rounding value carries a relative error of a few 2^-24,
which can move a value lying within that distance of a rounding midpoint
to the other neighbour; anything further off fails)."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, rmsnorm
from tests._gpu import dev16, host
from workloads import norm_inputs

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


def check(m, d, seed, sigma=0.01, delta=1e-6, inplace=False, noise=True):
    x, w = norm_inputs(m, d, seed)
    z = aqn.sample(seed, 5, 0, sigma, d) if noise else None
    xd, wd = dev16(x), dev16(w)
    zd = torch.from_numpy(z).to("cuda:0") if noise else None
    out = xd if inplace else None
    y = q.qerl_rmsnorm_noisy(xd, wd, zd, delta, out=out)
    torch.cuda.synchronize()
    got = formats.bf16_bits_to_f64(host(y).reshape(m, d))
    ref = rmsnorm.rmsnorm_noisy(x, w, z, delta)
    err = np.abs(got - ref)
    bad = err > bf16_ulp(ref)
    print(f"rmsnorm m={m} d={d} seed={seed} max_err_in_ulp="
          f"{float(np.max(err / np.maximum(bf16_ulp(ref), 1e-300))):.3f}", flush=True)
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])


@pytest.mark.parametrize("m,d", [(1, 8), (3, 40), (5, 520), (64, 3584), (7, 5120),
                                 (4096, 3584)])
def test_rmsnorm_parity(m, d):
    check(m, d, seed=m + d)


def test_rmsnorm_long_rows_two_passes():
    # more than 640 chunks per row: the grouped path that re-reads the row
    check(5, 8200, seed=11)
    check(2, 27648, seed=12)


def test_rmsnorm_no_noise_inplace_and_zero_delta():
    check(9, 1024, seed=13, noise=False)
    check(6, 3584, seed=14, inplace=True)
    check(4, 256, seed=15, delta=0.0)


def test_rmsnorm_zero_noise_is_plain_rmsnorm_bitwise():
    x, w = norm_inputs(16, 2048, 16)
    xd, wd = dev16(x), dev16(w)
    zero = torch.zeros(2048, dtype=torch.float32, device="cuda:0")
    a = q.qerl_rmsnorm_noisy(xd, wd, None)
    b = q.qerl_rmsnorm_noisy(xd, wd, zero)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
