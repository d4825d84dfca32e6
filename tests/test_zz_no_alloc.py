"""The entry point that allocates nothing (qerl_linear_decode_noalloc),
called through the C ABI: bit-identical to qerl_linear_decode with a
workspace, on two calls in a row (the second smaller, so it runs on what
the first left in the library's scratch), and the size limit refused
before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from tests._gpu import dev16, host
from workloads import make_layer

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402

lib = q.lib
P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None


def layer(m, n, k, r, seed):
    L = make_layer(m, n, k, r, seed=seed, outlier_frac=1e-3, call_id=3)
    codes, scales, S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
    z = q.qerl_aqn_sample(L.seed, 0, 3, 1e-2, k, device="cuda:0")
    return dict(x=dev16(L.x), codes=codes, scales=scales, S=S, z=z, m=m, n=n, k=k, r=r,
                a=dev16(L.a) if r else None, b=dev16(L.b) if r else None)


def call_both(d):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    m, n, k, r = d["m"], d["n"], d["k"], d["r"]
    y0 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    ws = q.workspace(m, n, k, r, "cuda:0")
    assert lib.qerl_linear_decode(P(d["x"]), m, P(d["codes"]), P(d["scales"]), P(d["S"]), n, k,
                                  P(d["a"]), P(d["b"]), r, 2.0, P(d["z"]), P(y0), P(ws),
                                  ws.numel(), st) == 0
    assert lib.qerl_linear_decode_noalloc(P(d["x"]), m, P(d["codes"]), P(d["scales"]), P(d["S"]),
                                          n, k, P(d["a"]), P(d["b"]), r, 2.0, P(d["z"]), P(y1),
                                          st) == 0
    torch.cuda.synchronize()
    return host(y0), host(y1)


def test_noalloc_matches_workspace_call_twice():
    big = layer(128, 2048, 5120, 64, seed=71)       # 128-token kernel, split K
    small = layer(17, 300, 1024, 8, seed=72)        # LDS-staged kernel, smaller scratch use
    for d in (big, small):
        y0, y1 = call_both(d)
        assert np.array_equal(y0, y1)


def test_noalloc_size_limit():
    limit = lib.qerl_linear_noalloc_scratch_bytes()
    assert limit == 64 << 20
    # a shape whose workspace exceeds the array: refused, y untouched
    m, n, k = 8192, 64, 8192
    assert lib.qerl_linear_workspace_bytes(m, n, k, 0) > limit
    fake = ctypes.c_void_p(0x10000)
    y = torch.full((1,), 7, dtype=torch.int16, device="cuda:0")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.qerl_linear_decode_noalloc(fake, m, fake, fake, fake, n, k, None, None, 0, 0.0,
                                          None, P(y), st) == 5
    torch.cuda.synchronize()
    assert int(y.item()) == 7
