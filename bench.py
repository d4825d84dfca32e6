"""Benchmark of the NVFP4 + LoRA + AQN linear layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]

A step is one rollout decode pass through a Qwen2.5-7B-shaped MLP block
with M = 64 tokens (8 prompts x 8 samples): for each of the fused gate/up
layer W [37888, 3584] and the down layer W [3584, 18944] (NVFP4, LoRA rank
32, s = 2), draw the layer's AQN noise vector for stage 1 of 10 and run
the linear layer (noisy activations, LoRA-down, NVFP4 contraction, LoRA-up
epilogue).  The noise vectors do not depend on the activations, so they
are drawn a few steps ahead on a second stream while earlier steps run.
The weights are quantized once before timing (the pages load the
quantized model once); the quantizer is timed on its own.  Six copies
of the quantized weights (684 MB) are used in rotation so that the 256 MB
Infinity Cache cannot serve them; inputs are resident in HBM before the
timed region.

Printed: one JSON line.  `value` = decode weight-stream GB/s (algorithmic
bytes of the step / step time); `roofline` = the decode contraction kernel
of the gate/up layer, timed alone with HIP events on its launch stream;
`mxfp4_decode` = the gate/up contraction on the weight quantized to MXFP4
(general and power-of-two dequantization);
`mlp_chain` = the same weights run as one chained feed-forward block (noisy
RMSNorm -> gate/up -> SiLU(gate) * up -> down) per step;
`prefill` = the 4096-token prefill of the Qwen2.5-7B qkv and down layers
in TFLOP/s; `rmsnorm` = the noisy RMSNorm producer on the 7B hidden size
(GB/s at 4096 rows, microseconds at 64 rows); `quantizer` = bulk
quantization GB/s; `cpu_baseline` = the oracle on the host cores on a
bounded slice of the same step.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=6)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chain", action="store_true")
    ap.add_argument("--profile", nargs="?", const="decode",
                    choices=("decode", "prefill", "rmsnorm", "backward", "chain", "mxfp4"),
                    help="profiling pass for rocprofv3, no timing and no JSON line: "
                         "'decode' runs one plain device copy of COPY_BYTES (counter "
                         "calibration) and PROFILE_LAUNCHES gate/up decode contractions; "
                         "'prefill' runs one prepare and three prefill GEMMs on each of "
                         "the 7B qkv and down layers at M=4096; 'rmsnorm' runs one "
                         "plain device copy (counter calibration) and 20 noisy RMSNorms "
                         "of 4096 x 3584 rows on rotated inputs; 'backward' runs one plain "
                         "device copy (counter calibration) and three backward calls (dx, "
                         "dA, dB) of the 7B down layer at M=4096; "
                         "'chain' runs PROFILE_LAUNCHES chained decode feed-forward steps "
                         "(noisy RMSNorm, gate/up, down on SwiGLU of the gate/up output); "
                         "'mxfp4' runs "
                         "PROFILE_LAUNCHES gate/up contractions on the MXFP4 weight with "
                         "the general and then with the power-of-two dequantization")
    return ap.parse_args()


COPY_BYTES = 512 << 20         # calibration copy of the profiling pass
PROFILE_LAUNCHES = 50          # gate/up contractions in the profiling pass


def linear_bytes(m, n, k, r):
    """Algorithmic bytes of one linear call: NVFP4 codes + scales, x, y,
    LoRA A and B (bf16), noise vector (fp32)."""
    return 0.5625 * n * k + 2 * m * k + 2 * m * n + 2 * r * (k + n) + 4 * k


def main_kernel_bytes(m, n, k, r):
    """Algorithmic bytes of the decode contraction kernel alone: codes +
    scales, x_t (bf16), y, the LoRA B factor and t = s x_t A^T (bf16)."""
    return 0.5625 * n * k + 2 * m * k + 2 * m * n + 2 * r * n + 2 * m * r


def linear_flops(m, n, k, r):
    return 2.0 * m * n * k + 2.0 * m * r * (k + n)


# Noise ring of the decode step: slots, steps sampled ahead, refill period.
# Slot safety: a refill at step i writes the slots of steps i + AHEAD - EVERY
# + 1 .. i + AHEAD after steps <= i - EVERY finished; the steps that may
# still read a slot are i - EVERY + 1 .. i + AHEAD - EVERY, so RING must
# exceed AHEAD + EVERY - 1.
NOISE_RING, NOISE_AHEAD, NOISE_EVERY = 12, 6, 4
assert NOISE_RING > NOISE_AHEAD + NOISE_EVERY - 1

# Sources of the decode contraction kernel timed for the roofline; the
# committed counter summary is only used while their digest is unchanged.
DECODE_SOURCES = ("decode_lds.h", "qerl_device.h", "decode.hip")


def source_digest(*names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "nvfp4_weight_quantized_qerl_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def profile_prefill(q, pc, make_layer, to_dev, dev):
    """Profiling pass of the prefill GEMM: per 7B layer at M=4096, one
    qerl_linear_prepare and three qerl_linear_prefill_prepared launches."""
    import torch
    psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
    for i, s in enumerate(pc.layers):
        L = make_layer(pc.m, s.n, s.k, pc.r, seed=11 + i, stage=pc.stage, call_id=i)
        x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
        codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
        del w
        z = q.qerl_aqn_sample(L.seed, 0, i, psig, s.k, device=dev)
        ws = q.workspace(pc.m, s.n, s.k, pc.r, dev)
        y = torch.empty((pc.m, s.n), dtype=torch.bfloat16, device=dev)
        q.qerl_linear_prepare(x, s.n, a, pc.lora_scale, z, ws)
        for _ in range(3):
            q.qerl_linear_prefill_prepared(pc.m, codes, scales, S, s.k, b, y, ws)
        torch.cuda.synchronize()
        del x, a, b, codes, scales, ws, y
    print("profile pass done: prefill_7b qkv and down, 3 GEMMs each")


def profile_rmsnorm(q, to_dev, dev, m=4096, d=3584, copies=10, launches=20):
    """Profiling pass of the noisy RMSNorm: one plain copy of COPY_BYTES
    (counter calibration), then `launches` calls on rotated input copies."""
    import torch
    from workloads import norm_inputs
    src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    x, w = norm_inputs(m, d, seed=31)
    wd = to_dev(w)
    xs = [to_dev(x) for _ in range(copies)]
    ys = [torch.empty_like(xs[0]) for _ in range(copies)]
    z = q.qerl_aqn_sample(31, 0, 0, 1e-2, d, device=dev)
    for i in range(launches):
        q.qerl_rmsnorm_noisy(xs[i % copies], wd, z, 1e-6, out=ys[i % copies])
    torch.cuda.synchronize()
    print(f"profile pass done: copy {COPY_BYTES} B, {launches} noisy RMSNorms {m}x{d}")


def profile_backward(q, pc, make_layer, to_dev, dev, calls=3):
    """Profiling pass of the backward: one plain copy of COPY_BYTES (counter
    calibration), then `calls` qerl_linear_backward calls (dx, dA, dB) of
    the 7B down layer at M=4096, r=32."""
    import torch
    from workloads import normal_bf16
    src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    s_dn = pc.layers[1]
    L = make_layer(pc.m, s_dn.n, s_dn.k, pc.r, seed=12, stage=pc.stage, call_id=1)
    x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
    codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
    del w
    psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
    z = q.qerl_aqn_sample(L.seed, 0, 1, psig, s_dn.k, device=dev)
    dy = to_dev(normal_bf16((pc.m, s_dn.n), 1.0, 12050))
    for _ in range(calls):
        q.qerl_linear_backward(dy, x, codes, scales, S, a, b, pc.lora_scale, z)
    torch.cuda.synchronize()
    print(f"profile pass done: {calls} backward calls of the 7B down layer at M={pc.m}")


def make_chain(q, layers, cfg, to_dev, dev, sigma, copies):
    """The 7B weights as one chained decode feed-forward block: noisy RMSNorm
    (Eq. 10, noise of the gate/up group) -> fused gate/up layer (no noise of
    its own) -> down layer (its own noise) on SiLU(gate) * up, which its
    prepare forms from the gate/up output (qerl_linear_decode_swiglu).  The
    two noise vectors are drawn here, before any timing.  Returns (step
    function, algorithmic bytes of one step)."""
    from workloads import norm_inputs
    M, R = cfg.m, cfg.r
    gu_l, dn_l = layers
    d_model, d_inter = gu_l["k"], dn_l["k"]
    xres_bits, wn_bits = norm_inputs(M, d_model, seed=41)
    xres, wnorm = to_dev(xres_bits), to_dev(wn_bits)
    z_gu = q.qerl_aqn_sample(41, 0, 0, sigma, d_model, device=dev)
    z_dn = q.qerl_aqn_sample(41, 0, 1, sigma, d_inter, device=dev)
    import torch
    h = torch.empty((M, d_model), dtype=torch.bfloat16, device=dev)

    def chain_step(i):
        cg, sg = gu_l["rot"][i % copies]
        cd, sd = dn_l["rot"][i % copies]
        q.qerl_rmsnorm_noisy(xres, wnorm, z_gu, 1e-6, out=h)
        q.qerl_linear_decode(h, cg, sg, gu_l["S"], gu_l["a"], gu_l["b"], cfg.lora_scale,
                             None, workspace=gu_l["ws"], y=gu_l["y"])
        q.qerl_linear_decode_swiglu(gu_l["y"], cd, sd, dn_l["S"], dn_l["a"], dn_l["b"],
                                    cfg.lora_scale, z_dn, workspace=dn_l["ws"], y=dn_l["y"])

    chain_bytes = (4 * M * d_model + 6 * d_model
                   + linear_bytes(M, gu_l["n"], d_model, R) - 4 * d_model
                   + 2 * M * d_inter               # the down layer reads gate and up
                   + linear_bytes(M, dn_l["n"], d_inter, R))
    return chain_step, chain_bytes


def make_mxfp4(q, gl, cfg, make_layer, to_dev, copies, z):
    """The gate/up weight quantized to MXFP4 (E8M0 per 32) and re-expressed
    in the NVFP4 layout, rotated like the NVFP4 copies, with the layer's
    prepare run on noise z.  Returns (rotation, FP32 scale S, range flag)."""
    Lg = make_layer(cfg.m, gl["n"], gl["k"], cfg.r, seed=1, stage=cfg.stage,
                    outlier_frac=cfg.outlier_frac, call_id=0)
    mcodes, ms8, _ = q.qerl_quantize_mxfp4(to_dev(Lg.w))
    ms4, mg, mflag = q.qerl_mxfp4_to_nvfp4(mcodes, ms8)
    mrot = [(mcodes, ms4)] + [(mcodes.clone(), ms4.clone()) for _ in range(copies - 1)]
    q.qerl_linear_prepare(gl["x"], gl["n"], gl["a"], cfg.lora_scale, z, gl["ws"])
    return mrot, mg, mflag


def oracle_step_rate(cfg, layers, M, R, min_seconds=10.0, max_reps=20):
    """The oracle running the decode step on the host: per layer, sample z,
    dequantize the NVFP4 weight and evaluate the fp64 linear layer with the
    LoRA branch.  As on the GPU, the weights are quantized (by the oracle)
    before timing; the step is repeated until min_seconds have passed."""
    import threadpoolctl
    from oracle import aqn, formats, linear, nvfp4

    prepared = []
    for ly in layers:
        L = ly["L"]
        w = formats.bf16_bits_to_f64(L.w)
        S = nvfp4.global_scale(nvfp4.tensor_amax(w))
        codes, scales = nvfp4.encode_with_scale(w, S)
        del w
        prepared.append((L, codes, scales, S))
    sig = aqn.sigma(cfg.sigma_start, cfg.sigma_end, cfg.num_stages, cfg.stage)
    step_bytes = sum(linear_bytes(M, ly["n"], ly["k"], R) for ly in layers)
    reps, t0 = 0, time.perf_counter()
    while True:
        for li, (L, codes, scales, S) in enumerate(prepared):
            z = aqn.sample(L.seed, 0, 2 * reps + li, sig, L.x.shape[1])
            w_hat = nvfp4.dequantize(codes, scales, S)
            linear.linear(L.x, w_hat, z, L.a, L.b, cfg.lora_scale)
            del w_hat
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
            if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    return {"value": round(reps * step_bytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{reps} full decode step(s), both layers and all rows (noise "
                      f"sample, NVFP4 dequantization, fp64 linear with LoRA), {dt:.1f} s; "
                      "weights quantized by the oracle before timing; dequantization "
                      f"runs on one thread, the fp64 matmuls on {threads} BLAS threads "
                      f"of {len(os.sched_getaffinity(0))} host cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the layer "
              "would shard by output rows, with one scalar max of amax before quantizing "
              "and no other exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_weight_quantized_qerl_amd as q
    from workloads import CONFIGS, make_layer

    dev = "cuda:0"
    torch.cuda.set_device(0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    stream = torch.cuda.current_stream()

    if args.profile == "prefill":
        profile_prefill(q, CONFIGS["prefill_7b"], make_layer, to_dev, dev)
        return
    if args.profile == "rmsnorm":
        profile_rmsnorm(q, to_dev, dev)
        return
    if args.profile == "backward":
        profile_backward(q, CONFIGS["prefill_7b"], make_layer, to_dev, dev)
        return

    cfg = CONFIGS["decode_7b_mlp"]
    M, R = cfg.m, cfg.r
    layers = []
    for i, s in enumerate(cfg.layers):
        L = make_layer(M, s.n, s.k, R, seed=1 + i, stage=cfg.stage,
                       outlier_frac=cfg.outlier_frac, call_id=i)
        layers.append(dict(name=s.name, n=s.n, k=s.k, L=L, x=to_dev(L.x), w=to_dev(L.w),
                           a=to_dev(L.a), b=to_dev(L.b)))

    # ---- quantize once (timed on its own: bulk quantizer GB/s)
    torch.cuda.synchronize()
    qtimes = []
    for rep in range(3):
        t0 = time.perf_counter()
        for ly in layers:
            ly["codes"], ly["scales"], ly["S"], ly["flag"] = q.qerl_quantize_nvfp4(ly["w"])
        torch.cuda.synchronize()
        qtimes.append(time.perf_counter() - t0)
    q_elems = sum(ly["n"] * ly["k"] for ly in layers)
    q_bytes = 2.5625 * q_elems
    assert all(int(ly["flag"].item()) == 0 for ly in layers)

    sigma = q.qerl_aqn_sigma(cfg.sigma_start, cfg.sigma_end, cfg.num_stages, cfg.stage)
    copies = max(1, args.copies)
    for ly in layers:
        ly["rot"] = [(ly["codes"], ly["scales"])] + [
            (ly["codes"].clone(), ly["scales"].clone()) for _ in range(copies - 1)]
        ly["z"] = torch.empty(ly["k"], dtype=torch.float32, device=dev)
        ly["ws"] = q.workspace(M, ly["n"], ly["k"], R, dev)
        ly["y"] = torch.empty((M, ly["n"]), dtype=torch.bfloat16, device=dev)
        del ly["w"]
    torch.cuda.empty_cache()

    if args.profile == "chain":
        chain_step, _ = make_chain(q, layers, cfg, to_dev, dev, sigma, copies)
        for i in range(PROFILE_LAUNCHES):
            chain_step(i)
        torch.cuda.synchronize()
        print(f"profile pass done: {PROFILE_LAUNCHES} chained decode feed-forward steps")
        return
    if args.profile == "mxfp4":
        gl = layers[0]
        z = q.qerl_aqn_sample(gl["L"].seed, 0, 0, sigma, gl["k"], device=dev)
        mrot, mg, _ = make_mxfp4(q, gl, cfg, make_layer, to_dev, copies, z)
        for fn in (q.qerl_linear_decode_prepared, q.qerl_linear_decode_prepared_mxfp4):
            for i in range(PROFILE_LAUNCHES):
                fn(M, *mrot[i % copies], mg, gl["k"], gl["b"], gl["y"], gl["ws"])
        torch.cuda.synchronize()
        print(f"profile pass done: {PROFILE_LAUNCHES} MXFP4 gate/up contractions with each "
              "dequantization")
        return
    if args.profile:
        # Plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch
        # calibrate the counters of the contraction kernel below.
        src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        ly = layers[0]
        q.qerl_aqn_sample(ly["L"].seed, 0, 0, sigma, ly["k"], out=ly["z"])
        q.qerl_linear_prepare(ly["x"], ly["n"], ly["a"], cfg.lora_scale, ly["z"], ly["ws"])
        for i in range(PROFILE_LAUNCHES):
            c, s = ly["rot"][i % copies]
            q.qerl_linear_decode_prepared(M, c, s, ly["S"], ly["k"], ly["b"], ly["y"], ly["ws"])
        torch.cuda.synchronize()
        print(f"profile pass done: copy {COPY_BYTES} B, {PROFILE_LAUNCHES} gate/up contractions "
              f"({main_kernel_bytes(M, ly['n'], ly['k'], R):.0f} algorithmic B each)")
        return

    # The AQN noise of a forward pass does not depend on its activations, so a
    # second stream (default priority) samples the noise vectors a few steps
    # ahead into a ring of slots, and each step waits only for its own slot.
    # Every NOISE_EVERY steps the main stream marks its progress and the host,
    # before refilling slots, waits for the mark of NOISE_EVERY steps earlier:
    # no slot is rewritten while a queued step may still read it.  (A wait of
    # the side stream on an event of the main stream, each step, serialised
    # the queues on this runtime.)
    side = torch.cuda.Stream(device=dev)
    zring = [[torch.empty(ly["k"], dtype=torch.float32, device=dev) for ly in layers]
             for _ in range(NOISE_RING)]
    z_ready = [torch.cuda.Event() for _ in range(NOISE_RING)]
    marks = {}

    def sample(j):
        sl = j % NOISE_RING
        for li, ly in enumerate(layers):
            q.qerl_aqn_sample(ly["L"].seed, 0, 2 * j + li, sigma, ly["k"],
                              out=zring[sl][li], stream=side)
        z_ready[sl].record(side)

    def step(i):
        sl = i % NOISE_RING
        stream.wait_event(z_ready[sl])
        for li, ly in enumerate(layers):
            codes, scales = ly["rot"][i % copies]
            q.qerl_linear_decode(ly["x"], codes, scales, ly["S"], ly["a"], ly["b"],
                                 cfg.lora_scale, zring[sl][li], workspace=ly["ws"], y=ly["y"])
        if i % NOISE_EVERY == NOISE_EVERY - 1:
            mark = torch.cuda.Event()
            mark.record(stream)
            marks[i] = mark
            old = marks.pop(i - NOISE_EVERY, None)
            if old is not None:
                old.synchronize()        # steps <= i - NOISE_EVERY are done
            for j in range(i + NOISE_AHEAD - NOISE_EVERY + 1, i + NOISE_AHEAD + 1):
                sample(j)

    for j in range(NOISE_AHEAD):
        sample(j)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = 1e3 * dt / args.steps
    step_bytes = sum(linear_bytes(M, ly["n"], ly["k"], R) for ly in layers)
    value = step_bytes / (dt / args.steps) / 1e9

    # ---- the same 7B weights as one chained decode feed-forward block: noisy
    # RMSNorm (Eq. 10, noise of the gate/up group) -> fused gate/up layer (no
    # noise of its own) -> SiLU(gate) * up -> down layer (its own noise).  The
    # two noise vectors are drawn before timing (the step above draws them on
    # a second stream, off its critical path).
    chain = None
    if not args.no_chain:
        chain_step, chain_bytes = make_chain(q, layers, cfg, to_dev, dev, sigma, copies)
        for i in range(args.warmup):
            chain_step(i)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(args.steps):
            chain_step(i)
        c1.record(stream)
        c1.synchronize()
        t_chain = c0.elapsed_time(c1) / 1e3 / args.steps
        chain = {"workload": "decode_7b_mlp chained: noisy RMSNorm -> gate/up -> down on "
                             "SiLU(gate)*up (formed in the down layer's prepare), M=64",
                 "us_per_step": round(t_chain * 1e6, 2),
                 "GB_per_s": round(chain_bytes / t_chain / 1e9, 1),
                 "frac_hbm": round(chain_bytes / t_chain / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- the gate/up weight as MXFP4 (E8M0 per 32) in the NVFP4 layout: the
    # contraction with the general dequantization and with the power-of-two
    # one, same rotation and workspace as the NVFP4 roofline pass below
    mx = None
    if not args.no_chain:
        gl = layers[0]
        mrot, mg, mflag = make_mxfp4(q, gl, cfg, make_layer, to_dev, copies, zring[0][0])
        mx = {"workload": "gate/up 37888x3584 MXFP4 weight in the NVFP4 layout, M=64, r=32",
              "range_flag": int(mflag.item())}
        mx_bytes = main_kernel_bytes(M, gl["n"], gl["k"], R)
        # three interleaved rounds, median per variant (box noise is ~±5%)
        mx_t = {"general_us": [], "pow2_us": []}
        for _ in range(3):
            for name, fn in (("general_us", q.qerl_linear_decode_prepared),
                             ("pow2_us", q.qerl_linear_decode_prepared_mxfp4)):
                for i in range(5):
                    fn(M, *mrot[i % copies], mg, gl["k"], gl["b"], gl["y"], gl["ws"])
                m0 = torch.cuda.Event(enable_timing=True)
                m1 = torch.cuda.Event(enable_timing=True)
                m0.record(stream)
                for i in range(max(20, args.steps)):
                    fn(M, *mrot[i % copies], mg, gl["k"], gl["b"], gl["y"], gl["ws"])
                m1.record(stream)
                m1.synchronize()
                mx_t[name].append(m0.elapsed_time(m1) * 1e3 / max(20, args.steps))
        for name, v in mx_t.items():
            mx[name] = round(sorted(v)[1], 2)
        mx["pow2_GB_per_s"] = round(mx_bytes / (mx["pow2_us"] * 1e-6) / 1e9, 1)
        del mrot

    # ---- dominant kernel alone: gate/up contraction, HIP events on its stream
    ly = layers[0]
    q.qerl_linear_prepare(ly["x"], ly["n"], ly["a"], cfg.lora_scale, zring[0][0], ly["ws"])
    reps = max(20, args.steps)
    for i in range(5):
        c, s = ly["rot"][i % copies]
        q.qerl_linear_decode_prepared(M, c, s, ly["S"], ly["k"], ly["b"], ly["y"], ly["ws"])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(reps):
        c, s = ly["rot"][i % copies]
        q.qerl_linear_decode_prepared(M, c, s, ly["S"], ly["k"], ly["b"], ly["y"], ly["ws"])
    ev1.record(stream)
    ev1.synchronize()
    kern_s = ev0.elapsed_time(ev1) / 1e3 / reps
    kbytes = main_kernel_bytes(M, ly["n"], ly["k"], R)
    achieved = kbytes / kern_s / 1e9
    digest = source_digest(*DECODE_SOURCES)
    traffic = measured_traffic("decode_main_gate_up_7b", digest)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "decode_main (gate/up 37888x3584, M=64, r=32)",
                "avg_launch_us": round(kern_s * 1e6, 2), "bytes_per_launch": kbytes}

    # ---- prefill (Qwen2.5-7B qkv and down, 4096 tokens): TFLOP/s, for the
    # whole call (prepare + GEMM) and for the GEMM kernel alone
    prefill = None
    backward = None
    if not args.no_prefill:
        pc = CONFIGS["prefill_7b"]
        psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
        per_layer, t_full, t_main, pflops = [], 0.0, 0.0, 0.0
        for i, s in enumerate(pc.layers):
            L = make_layer(pc.m, s.n, s.k, pc.r, seed=11 + i, stage=pc.stage, call_id=i)
            x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
            codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
            del w
            z = q.qerl_aqn_sample(L.seed, 0, i, psig, s.k, device=dev)
            ws = q.workspace(pc.m, s.n, s.k, pc.r, dev)
            y = torch.empty((pc.m, s.n), dtype=torch.bfloat16, device=dev)

            def timed(fn, reps=5):
                for _ in range(2):
                    fn()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                e1.synchronize()
                return e0.elapsed_time(e1) / 1e3 / reps

            tf = timed(lambda: q.qerl_linear_prefill(x, codes, scales, S, a, b, pc.lora_scale,
                                                      z, workspace=ws, y=y))
            q.qerl_linear_prepare(x, s.n, a, pc.lora_scale, z, ws)
            tm = timed(lambda: q.qerl_linear_prefill_prepared(pc.m, codes, scales, S, s.k, b,
                                                               y, ws))
            fl = linear_flops(pc.m, s.n, s.k, pc.r)
            per_layer.append({"layer": f"{s.name} {s.n}x{s.k}",
                              "tflops": round(fl / tf / 1e12, 1),
                              "gemm_tflops": round(fl / tm / 1e12, 1),
                              "ms": round(1e3 * tf, 3), "gemm_ms": round(1e3 * tm, 3)})
            t_full += tf
            t_main += tm
            pflops += fl
            del x, a, b, codes, scales, ws, y
        # backward through the frozen NVFP4 weight of the 7B down layer at the
        # same 4096 tokens: dx, dA and dB
        s_dn = pc.layers[1]
        L = make_layer(pc.m, s_dn.n, s_dn.k, pc.r, seed=12, stage=pc.stage, call_id=1)
        x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
        codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
        del w
        z = q.qerl_aqn_sample(L.seed, 0, 1, psig, s_dn.k, device=dev)
        from workloads import normal_bf16
        dy = to_dev(normal_bf16((pc.m, s_dn.n), 1.0, 12050))
        bws = torch.empty(q.lib.qerl_linear_backward_workspace_bytes(pc.m, s_dn.n, s_dn.k, pc.r),
                          dtype=torch.uint8, device=dev)
        tb = timed(lambda: q.qerl_linear_backward(dy, x, codes, scales, S, a, b, pc.lora_scale,
                                                  z, workspace=bws), reps=3)
        mm, nn, kk, rr = pc.m, s_dn.n, s_dn.k, pc.r
        bflops = (2.0 * mm * nn * kk          # dy W_hat
                  + 2.0 * mm * rr * kk * 3     # t = x_t A^T, gs A, dA
                  + 2.0 * mm * nn * rr * 2)    # gs = dy B, dB
        backward = {"workload": f"backward of the 7B down layer: dy {mm}x{nn}, W {nn}x{kk} "
                                f"NVFP4, r={rr} (dx, dA, dB)",
                    "ms": round(1e3 * tb, 3), "tflops": round(bflops / tb / 1e12, 1),
                    "frac_bf16_peak": round(bflops / tb / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del x, a, b, codes, scales, dy, bws
        prefill = {"workload": "prefill_7b (qkv 4608x3584 + down 3584x18944, M=4096, r=32)",
                   "tflops": round(pflops / t_full / 1e12, 1),
                   "gemm_tflops": round(pflops / t_main / 1e12, 1),
                   "ms": round(1e3 * t_full, 3),
                   "frac_bf16_peak": round(pflops / t_full / 1e12 / BF16_PEAK_TFLOPS, 4),
                   "gemm_frac_bf16_peak": round(pflops / t_main / 1e12 / BF16_PEAK_TFLOPS, 4),
                   "layers": per_layer}

    # ---- noisy RMSNorm producer (Eq. 10) on the 7B hidden size: the 4096-token
    # prefill rows (HBM-bound; copies rotated past the Infinity Cache) and the
    # 64 decode rows (latency-bound)
    rmsnorm = None
    if not args.no_prefill:
        from workloads import norm_inputs
        rmsnorm = []
        for m, d, copies_n in ((4096, 3584, 10), (64, 3584, 1)):
            xs_, ws_ = norm_inputs(m, d, seed=31)
            wd = to_dev(ws_)
            xcopies = [to_dev(xs_) for _ in range(copies_n)]
            ycopies = [torch.empty_like(xcopies[0]) for _ in range(copies_n)]
            zd = q.qerl_aqn_sample(31, 0, 0, sigma, d, device=dev)
            run = lambda i: q.qerl_rmsnorm_noisy(xcopies[i % copies_n], wd, zd, 1e-6,
                                                 out=ycopies[i % copies_n])
            for i in range(5):
                run(i)
            reps = 50
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                run(i)
            e1.record(stream)
            e1.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / reps
            nbytes = 4 * m * d + 2 * d + 4 * d
            rmsnorm.append({"workload": f"noisy RMSNorm {m}x{d} (Qwen2.5-7B hidden)",
                            "us": round(t * 1e6, 2), "GB_per_s": round(nbytes / t / 1e9, 1),
                            "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes": nbytes})
            del xcopies, ycopies

    # ---- oracle on the host cores: the same step, weights quantized beforehand
    cpu = None
    if not args.no_cpu:
        cpu = oracle_step_rate(cfg, layers, M, R)

    out = {
        "metric": "NVFP4+LoRA linear: decode weight-stream GB/s and prefill TFLOP/s, % roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (NVFP4 weights)", "data": "synthetic",
        "config": {"workload": "decode_7b_mlp: Qwen2.5-7B-shaped MLP, M=64 (8 prompts x 8 "
                               "samples), gate/up 37888x3584 + down 3584x18944 NVFP4, LoRA "
                               "r=32, AQN stage 1/10", "global_batch": M,
                   "weight_copies_rotated": copies, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "prefill": prefill,
        "rmsnorm": rmsnorm,
        "mlp_chain": chain,
        "backward": backward,
        "mxfp4_decode": mx,
        "quantizer": {"GB_per_s": round(q_bytes / min(qtimes) / 1e9, 1),
                      "elements": q_elems, "bytes_per_elem": 2.5625},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
