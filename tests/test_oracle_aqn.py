"""Pins for oracle.aqn: page-printed schedule facts, numpy's own Philox
bit generator, closed-form Box-Muller values and normal statistics."""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import aqn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLDEN, "aqn_schedule.json")))


def ulp(x):
    return np.spacing(abs(x))


def test_schedule_endpoints_and_stage0():
    s0, s1, K = G["sigma_start"], G["sigma_end"], G["num_stages"]
    assert aqn.sigma(s0, s1, K, 0) == G["stage0_sigma"]
    assert aqn.sigma(s0, s1, K, 1) == s0
    assert abs(aqn.sigma(s0, s1, K, K) - s1) <= 2 * ulp(s1)


def test_schedule_constant_ratio_and_monotone():
    s0, s1, K = G["sigma_start"], G["sigma_end"], G["num_stages"]
    sig = [aqn.sigma(s0, s1, K, k) for k in range(1, K + 1)]
    ratio = (s1 / s0) ** (1.0 / (K - 1))
    for a, b in zip(sig, sig[1:]):
        assert b < a
        assert abs(b / a - ratio) < 1e-14
    # geometric interpolation: log sigma is linear in k
    logs = np.log(sig)
    assert np.allclose(np.diff(logs, 2), 0.0, atol=1e-13)
    # stage 3 and the mid-schedule stage used by the workloads
    assert abs(sig[2] - s0 * ratio ** 2) < 1e-17
    assert abs(sig[2] - 5.139042664e-3) < 1e-12
    assert abs(sig[4] - 2.640975950e-3) < 1e-12


def test_schedule_single_stage_and_errors():
    assert aqn.sigma(1e-2, 5e-4, 1, 1) == 1e-2
    for bad in [(1e-2, 5e-4, 10, 11), (1e-2, 5e-4, 0, 0), (0.0, 5e-4, 10, 2),
                (1e-2, -1.0, 10, 2), (1e-2, 5e-4, 10, -1)]:
        with pytest.raises(ValueError):
            aqn.sigma(*bad)


def _numpy_philox_block(counter, key):
    """Block at `counter` from numpy's Philox (4x64, 10 rounds), which
    increments its 256-bit counter before producing each block."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & aqn.MASK64 for i in range(4)],
                     dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return tuple(int(v) for v in bg.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)), ((1, 0, 0, 0), (1, 2)),
    ((7, 3, 0, 0), (12345, 6)), ((0, 0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1)),
    ((2 ** 64 - 1, 2 ** 32, 0, 0), (0xDEADBEEF, 0)),
    ((123456789, 987654321, 5, 9), (42, 43))])
def test_philox_matches_numpy_bitgenerator(counter, key):
    assert aqn.philox4x64(counter, key) == _numpy_philox_block(counter, key)


def test_box_muller_closed_forms():
    top = (2 ** 53 - 1) << 11                  # u1 = 1 -> radius 0
    assert aqn.box_muller_pair(top, 12345 << 11) == (0.0, 0.0)
    r_a = 0                                     # u1 = 2**-53
    rad = math.sqrt(-2.0 * math.log(2.0 ** -53))
    n0, n1 = aqn.box_muller_pair(r_a, 0)        # u2 = 0 -> angle 0
    assert n0 == rad and n1 == 0.0
    n0, n1 = aqn.box_muller_pair(r_a, (2 ** 51) << 11)   # u2 = 1/4
    assert abs(n0) < 1e-15 * rad and n1 == pytest.approx(rad, rel=1e-15)
    n0, n1 = aqn.box_muller_pair(r_a, (2 ** 52) << 11)   # u2 = 1/2
    assert n0 == pytest.approx(-rad, rel=1e-15) and abs(n1) < 1e-15 * rad


def test_noise_statistics():
    d = 1 << 18
    n = aqn.standard_normals(seed=2024, stream_id=1, call_id=0, d=d)
    assert abs(n.mean()) < 5.0 / math.sqrt(d)
    assert abs(n.std() - 1.0) < 5.0 / math.sqrt(2 * d)
    assert stats.kstest(n, "norm").pvalue > 1e-3
    # the four lanes of a counter block are each standard normal
    for i in range(4):
        lane = n[i::4]
        assert abs(lane.mean()) < 5.0 / math.sqrt(lane.size)
        assert abs(lane.std() - 1.0) < 5.0 / math.sqrt(2 * lane.size)


def test_noise_reproducible_and_independent():
    a = aqn.standard_normals(1, 0, 0, 4096)
    b = aqn.standard_normals(1, 0, 0, 4096)
    c = aqn.standard_normals(1, 0, 1, 4096)
    d = aqn.standard_normals(1, 1, 0, 4096)
    e = aqn.standard_normals(2, 0, 0, 4096)
    assert np.array_equal(a, b)
    for other in (c, d, e):
        assert abs(np.corrcoef(a, other)[0, 1]) < 5.0 / math.sqrt(4096)
    # prefix property: element j depends only on (seed, stream, call, j)
    assert np.array_equal(aqn.standard_normals(1, 0, 0, 13), a[:13])


def test_sample_is_sigma_times_normal_in_fp32():
    sig = aqn.sigma(1e-2, 5e-4, 10, 3)
    z = aqn.sample(0, 0, 0, sig, 256)
    n = aqn.standard_normals(0, 0, 0, 256)
    assert z.dtype == np.float32
    assert np.array_equal(z, (sig * n).astype(np.float32))
    assert np.all(aqn.sample(0, 0, 0, 0.0, 256) == 0.0)


# ---- the four decay schedules compared on the pages (linear, exponential,
# cosine, logarithmic) [QeRL summary, §3.4, "Why exponential decay"]

def test_every_schedule_runs_from_start_to_end():
    for mode in aqn.SCHEDULES:
        for K in (2, 5, 10):
            assert aqn.sigma_schedule(mode, 1e-2, 5e-4, K, 1) == pytest.approx(1e-2, rel=1e-15)
            assert aqn.sigma_schedule(mode, 1e-2, 5e-4, K, K) == pytest.approx(5e-4, rel=1e-13)
            assert aqn.sigma_schedule(mode, 1e-2, 5e-4, K, 0) == 0.0
        assert aqn.sigma_schedule(mode, 1e-2, 5e-4, 1, 1) == 1e-2


def test_schedules_decrease_monotonically():
    for mode in aqn.SCHEDULES:
        vals = [aqn.sigma_schedule(mode, 1e-2, 5e-4, 10, k) for k in range(1, 11)]
        assert all(a > b for a, b in zip(vals, vals[1:])), mode


def test_schedule_midpoints():
    s0, s1 = 1e-2, 5e-4
    mean = 0.5 * (s0 + s1)
    # K = 9: stage 5 is half way in t = (k-1)/(K-1); linear and cosine pass
    # through the arithmetic mean there, exponential through the geometric
    # mean; the logarithmic schedule is half way at k = 3 (ln 3 / ln 9 = 1/2).
    assert aqn.sigma_schedule("linear", s0, s1, 9, 5) == pytest.approx(mean, rel=1e-15)
    assert aqn.sigma_schedule("cosine", s0, s1, 9, 5) == pytest.approx(mean, rel=1e-15)
    assert aqn.sigma_schedule("exponential", s0, s1, 9, 5) == pytest.approx((s0 * s1) ** 0.5, rel=1e-14)
    assert aqn.sigma_schedule("logarithmic", s0, s1, 9, 3) == pytest.approx(mean, rel=1e-14)


def test_linear_schedule_steps_are_equal_and_log_drops_fastest():
    lin = [aqn.sigma_schedule("linear", 1e-2, 5e-4, 10, k) for k in range(1, 11)]
    steps = [a - b for a, b in zip(lin, lin[1:])]
    assert max(steps) - min(steps) < 1e-17
    assert steps[0] == pytest.approx((1e-2 - 5e-4) / 9, rel=1e-12)
    # the first step is largest for the logarithmic schedule (sharp initial drop)
    first = {m: 1e-2 - aqn.sigma_schedule(m, 1e-2, 5e-4, 10, 2) for m in aqn.SCHEDULES}
    assert max(first, key=first.get) == "logarithmic"
    # the cosine schedule starts flat: its first step is the smallest
    assert min(first, key=first.get) == "cosine"
