"""GPU parity of the gated activation (qerl_swiglu) and of a chained
decode feed-forward block built from the library's calls:
noisy RMSNorm (Eq. 10) -> fused gate/up layer (no noise of its own) ->
SiLU(gate) * up -> down layer with its own noise vector.

Bars: SwiGLU outputs are faithful bf16 roundings of the fp64 value (one
bf16 ulp; the hardware exp and reciprocal and the fp32 products carry a few
2^-24, against the 2^-8 of a bf16 ulp).  Each call of the chain
returns bf16 (the interface of every call), so the oracle chain rounds to
bf16 (nearest even) at the same three points and is otherwise fp64; the
chain's output is then within the layer tolerance (max error 2e-2 of
max(|y*|, rms(y*))).  Without those roundings the oracle chain differs by
the compounded 2^-9 per-call roundings (about 1.7e-2 at this size), which
is printed for reference."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, linear, nvfp4, rmsnorm, swiglu
from tests._gpu import dev16, host
from workloads import make_layer, norm_inputs, normal_bf16

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402


def round_bf16(v):
    """fp64 -> nearest bf16 value, ties to even (normal range)."""
    mant, expo = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.rint(mant * 256.0) / 256.0, expo)


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


@pytest.mark.parametrize("m,d", [(1, 8), (3, 40), (64, 18944), (256, 13824)])
def test_swiglu_parity(m, d):
    gu = normal_bf16((m, 2 * d), 2.0, 70 + m)
    out = q.qerl_swiglu(dev16(gu))
    torch.cuda.synchronize()
    got = formats.bf16_bits_to_f64(host(out).reshape(m, d))
    ref = swiglu.swiglu(gu)
    err = np.abs(got - ref)
    print(f"swiglu m={m} d={d} max_err_in_ulp="
          f"{float(np.max(err / np.maximum(bf16_ulp(ref), 1e-300))):.3f}", flush=True)
    assert not (err > bf16_ulp(ref)).any()


def test_chained_decode_mlp():
    m, hidden, inter, r = 16, 512, 1024, 8
    x, w_norm = norm_inputs(m, hidden, seed=80)
    z_gu = aqn.sample(80, 0, 0, 1e-2, hidden)
    z_dn = aqn.sample(80, 0, 1, 1e-2, inter)
    Lgu = make_layer(m, 2 * inter, hidden, r, seed=81)
    Ldn = make_layer(m, hidden, inter, r, seed=82)
    dev = "cuda:0"
    # GPU chain: every step one library call
    cg, sg, Sg, _ = q.qerl_quantize_nvfp4(dev16(Lgu.w))
    cd, sd, Sd, _ = q.qerl_quantize_nvfp4(dev16(Ldn.w))
    zg, zd = torch.from_numpy(z_gu).to(dev), torch.from_numpy(z_dn).to(dev)
    h = q.qerl_rmsnorm_noisy(dev16(x), dev16(w_norm), zg, 1e-6)
    gu = q.qerl_linear_decode(h, cg, sg, Sg, dev16(Lgu.a), dev16(Lgu.b), 2.0, None)
    act = q.qerl_swiglu(gu)
    y = q.qerl_linear_decode(act, cd, sd, Sd, dev16(Ldn.a), dev16(Ldn.b), 2.0, zd)
    # the same down layer with the activation formed inside its prepare
    y_fused = q.qerl_linear_decode_swiglu(gu, cd, sd, Sd, dev16(Ldn.a), dev16(Ldn.b), 2.0, zd)
    torch.cuda.synchronize()
    assert torch.equal(y_fused, y)
    got = formats.bf16_bits_to_f64(host(y).reshape(m, hidden))
    # oracle chain in fp64, each call's output rounded to bf16 as the calls return it
    wg = nvfp4.dequantize(*nvfp4.quantize(Lgu.w))
    wd = nvfp4.dequantize(*nvfp4.quantize(Ldn.w))

    def chain(rnd):
        h_ref = rnd(rmsnorm.rmsnorm_noisy(x, w_norm, z_gu, 1e-6))
        gu_ref = rnd(linear.linear_values(h_ref, wg, None, Lgu.a, Lgu.b, 2.0))
        act_ref = rnd(swiglu.silu(gu_ref[:, :inter]) * gu_ref[:, inter:])
        return linear.linear_values(act_ref, wd, z_dn, Ldn.a, Ldn.b, 2.0)

    err = linear.max_rel_error(got, chain(round_bf16))
    err_unrounded = linear.max_rel_error(got, chain(lambda v: v))
    print(f"chained mlp max_rel_error={err:.4g} (vs the unrounded fp64 chain: "
          f"{err_unrounded:.4g})", flush=True)
    assert err <= 2e-2


@pytest.mark.parametrize("m,n,k,r,noise", [
    (5, 96, 160, 16, True),       # ragged m, one partial K chunk of the prepare
    (37, 128, 1024, 0, True),     # no LoRA branch (the elementwise x_t kernel)
    (64, 256, 512, 40, False),    # two rank groups, no noise
    (64, 3584, 18944, 32, True),  # the 7B down layer at 64 tokens
    (130, 64, 272, 8, True),      # two decode chunks of m, k % 256 != 0 (general kernel)
])
def test_decode_swiglu_is_swiglu_then_decode(m, n, k, r, noise):
    """qerl_linear_decode_swiglu(gate_up) == qerl_linear_decode(qerl_swiglu(gate_up)),
    bit for bit: both form bf16(SiLU(g) u) with the same fp32 arithmetic."""
    print(f"decode_swiglu m={m} n={n} k={k} r={r} noise={noise}", flush=True)
    L = make_layer(m, n, k, r, seed=90 + m)
    gu = dev16(normal_bf16((m, 2 * k), 2.0, 91 + m))
    c, s, S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
    z = q.qerl_aqn_sample(92, 0, m, 1e-2, k, device="cuda:0") if noise else None
    a = dev16(L.a) if r else None
    b = dev16(L.b) if r else None
    ref = q.qerl_linear_decode(q.qerl_swiglu(gu), c, s, S, a, b, 2.0, z)
    got = q.qerl_linear_decode_swiglu(gu, c, s, S, a, b, 2.0, z)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
