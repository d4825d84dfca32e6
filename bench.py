"""Benchmark of the NVFP4 + LoRA + AQN linear layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--only sweep]

Headline step: one rollout decode pass through a Qwen2.5-32B-shaped model
(hidden 5120, intermediate 27648, 40 q / 8 kv heads of dim 128): 64 layers x
{qkv [7168, 5120], o [5120, 5120], gate/up [55296, 5120], down [5120, 27648]}
of NVFP4 weights (17.55 GB, streamed once per step), M = 128 rollout tokens
(8 prompts x 16 samples), LoRA rank 64 (s = 2) on every projection, AQN
stage 1 of 10.  A step draws the step's 256 noise vectors (one per
projection and layer, call id 256 * step + 4 * layer + projection; four
batched launches) and runs the 256 linear calls (noisy activations,
LoRA-down, NVFP4 contraction, LoRA-up epilogue).  The weights are generated
and quantized on the device once before timing (the pages load the
quantized model once).  The calls are independent: each projection reads a
fixed synthetic activation of its input width.

Timing: W untimed warm-up steps, then K timed steps with a HIP event
between consecutive steps on the launch stream; `value` = algorithmic bytes
of a step / median step time (GB/s), with p10 / p90 beside it.  The same
protocol (median, p10, p90 of per-iteration events) is used for every
sub-measurement:
  `roofline`            the dominant kernel: the gate/up contraction of the
                        sweep (MFMA-bound at 128 tokens), timed alone;
  `decode_7b_mlp`       the 7B MLP at 64 tokens (gate/up + down, noise drawn
                        ahead on a second stream), its gate/up contraction
                        kernel, the chained feed-forward block and the MXFP4
                        weight;
  `decode_layer_7b`     a whole 7B decode layer at 64 tokens as a chain of calls
                        (noisy RMSNorm, q/k/v, attention stub, o, gate/up,
                        SiLU * up, down), with per-call and per-row noise;
  `prefill_7b`          4096-token prefill of the 7B qkv and down layers, and
                        the backward of the 7B down layer;
  `quantize_prefill_14b` bulk quantization of every linear weight of a
                        Qwen2.5-14B-shaped model (48 layers) and the
                        16384-token prefill through one layer's o, gate, up,
                        down;
  `rmsnorm`             the noisy RMSNorm producer;
  `cpu_baseline`        the oracle on the host cores on a labelled slice of
                        the headline step.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

COPY_BYTES = 512 << 20         # calibration copy of the profiling passes
PROFILE_LAUNCHES = 50          # contractions of a profiling pass

PARTS = ("sweep", "decode7b", "layer7b", "prefill7b", "q14b", "rmsnorm")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=6,
                    help="rotated weight copies of the 7B decode measurements")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", nargs="+", choices=PARTS, default=None,
                    help="run only these parts (the headline is always reported when run)")
    ap.add_argument("--profile", choices=("decode", "sweep32", "prefill", "rmsnorm", "backward",
                                          "chain", "mxfp4", "quant14b", "prefill14b"),
                    help="profiling pass for rocprofv3, no timing and no JSON line: "
                         "'decode' = one plain copy of COPY_BYTES (counter calibration) and "
                         "PROFILE_LAUNCHES 7B gate/up contractions at M=64; 'sweep32' = one "
                         "plain copy, 3 full 32B sweep steps, then PROFILE_LAUNCHES 32B gate/up "
                         "contractions at M=128; 'prefill' = per 7B layer at M=4096 one prepare "
                         "and three prefill GEMMs; 'rmsnorm' = one plain copy and 20 noisy "
                         "RMSNorms 4096x3584; 'backward' = one plain copy and three backward "
                         "calls of the 7B down layer at M=4096; 'chain' = PROFILE_LAUNCHES "
                         "chained 7B feed-forward steps; 'mxfp4' = PROFILE_LAUNCHES MXFP4 gate/up "
                         "contractions with each dequantization; 'quant14b' = one plain copy and "
                         "one bulk quantization of the 14B model; 'prefill14b' = per 14B layer "
                         "(o, gate, up, down) at M=16384 one prepare and three prefill GEMMs")
    return ap.parse_args()


# ----------------------------------------------------------------- figures
def linear_bytes(m, n, k, r):
    """Algorithmic bytes of one linear call: NVFP4 codes + scales, x, y,
    LoRA A and B (bf16), noise vector (fp32)."""
    return 0.5625 * n * k + 2 * m * k + 2 * m * n + 2 * r * (k + n) + 4 * k


def main_kernel_bytes(m, n, k, r):
    """Algorithmic bytes of the decode contraction alone: codes + scales,
    x_t (bf16), y, the LoRA B factor and t = s x_t A^T (bf16)."""
    return 0.5625 * n * k + 2 * m * k + 2 * m * n + 2 * r * n + 2 * m * r


def linear_flops(m, n, k, r):
    return 2.0 * m * n * k + 2.0 * m * r * (k + n)


def main_kernel_flops(m, n, k, r):
    """Flops of the contraction alone: x_t W^T and the LoRA-up t B^T."""
    return 2.0 * m * n * k + 2.0 * m * r * n


def stats_ms(times_ms):
    """median / p10 / p90 / mean of per-iteration times (ms)."""
    import numpy as np
    a = np.asarray(times_ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 5),
            "p10_ms": round(float(np.percentile(a, 10)), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5),
            "mean_ms": round(float(a.mean()), 5), "iters": int(a.size)}


def event_times(fn, iters, stream, warmup=3):
    """Per-iteration times (ms) of fn(i), i = 0..iters-1, from HIP events
    recorded between consecutive iterations on `stream` (after `warmup`
    untimed calls)."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(stream)
    for i in range(iters):
        fn(i)
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]


def batch_times(fn, stream, batches=10, per_batch=20, warmup=5):
    """Average time (ms) per call of fn(i) in each of `batches` batches of
    `per_batch` back-to-back calls, from HIP events around each batch on
    `stream` (an event between every two calls would add its own time to
    short kernels)."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
    ev[0].record(stream)
    for b in range(batches):
        for j in range(per_batch):
            fn(b * per_batch + j)
        ev[b + 1].record(stream)
    ev[-1].synchronize()
    return [ev[b].elapsed_time(ev[b + 1]) / per_batch for b in range(batches)]


def gpu_clock():
    """Current shader clock (MHz) as rocm-smi reports it, or None."""
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                             text=True, timeout=20).stdout
        data = json.loads(out[out.index("{"):])
    except Exception:          # rocm-smi missing or unparsable: no clock recorded
        return None
    for card in data.values():
        for key, val in card.items():
            if "sclk" in key.lower():
                digits = "".join(ch for ch in str(val) if ch.isdigit())
                if digits:
                    return int(digits)
    return None


# Sources of each decode contraction kernel and its launch; a committed
# counter summary is only used while their digest is unchanged.
M128_SOURCES = ("decode_m128.h", "decode_m128.hip", "qerl_device.h", "decode.hip")
LDS_SOURCES = ("decode_lds.h", "decode_lds_mt1.hip", "decode_lds_mt2.hip", "qerl_device.h",
               "decode.hip")


def source_digest(*names):
    h = hashlib.sha256()
    for name in names:
        path = os.path.join(ROOT, "nvfp4_weight_quantized_qerl_amd", "csrc", name)
        if os.path.exists(path):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def calibration_copy(dev):
    """One plain device copy of COPY_BYTES: its FETCH_SIZE / WRITE_SIZE
    calibrate the counters of the kernels profiled after it."""
    import torch
    src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def dev_normal(shape, std, gen, dev):
    """N(0, std^2) drawn in fp32 on the device from a seeded generator and
    rounded to bf16 (nearest even)."""
    import torch
    return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
            * std).to(torch.bfloat16)


def library_bf16_gemm_ms(m, n, k, dev, stream, gen, iters=10):
    """Median time (ms) of the vendor library's dense bf16 GEMM (torch.matmul,
    hipBLASLt on this image) at the same shape: x [m, k] N(0, 1) times a
    dense bf16 weight [k, n] N(0, 0.02^2), fp32 accumulation, no
    dequantization, no LoRA and four times the weight bytes.  A reference
    point for what a GEMM reaches on this machine with random data, not part of
    the path."""
    import torch
    x = dev_normal((m, k), 1.0, gen, dev)
    wt = dev_normal((k, n), 0.02, gen, dev)       # contiguous [k, n] right operand
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    st = stats_ms(event_times(lambda i: torch.matmul(x, wt, out=y), iters, stream))
    del x, wt, y
    return st["median_ms"]


# ------------------------------------------------- headline: the 32B sweep
class Sweep32:
    """The Qwen2.5-32B decode sweep (64 layers x 4 projections, M=128, r=64),
    generated and quantized on the device (seeded), held in the tiled layout
    of the 128-token kernel, with every call bound."""

    def __init__(self, q, cfg, dev, keep_host_layer0=False):
        import torch
        self.q, self.cfg, self.dev = q, cfg, dev
        M, R = cfg.m, cfg.r
        self.sigma = q.qerl_aqn_sigma(cfg.sigma_start, cfg.sigma_end, cfg.num_stages, cfg.stage)
        gen = torch.Generator(device=dev)
        gen.manual_seed(4000)
        self.shapes = cfg.layers                     # qkv, o, gate_up, down
        self.x = {}
        for s in self.shapes:
            if s.k not in self.x:
                self.x[s.k] = dev_normal((M, s.k), 1.0, gen, dev)
        self.z = [torch.empty((cfg.n_layers, s.k), dtype=torch.float32, device=dev)
                  for s in self.shapes]
        self.ws = [q.tiled_workspace(M, s.n, s.k, R, dev) for s in self.shapes]
        self.y = [torch.empty((M, s.n), dtype=torch.bfloat16, device=dev) for s in self.shapes]
        self.layers = []                             # [layer][proj] dict
        self.host_w0 = []
        flags = []
        for li in range(cfg.n_layers):
            row = []
            for p, s in enumerate(self.shapes):
                w = dev_normal((s.n, s.k), 0.02, gen, dev)
                codes, scales, S, flag = q.qerl_quantize_nvfp4(w)
                flags.append(flag)
                if li == 0 and keep_host_layer0:
                    self.host_w0.append(w[:512].view(torch.int16).cpu().numpy().view("uint16"))
                del w
                # held in the tiled layout of the 128-token kernel (re-laid once)
                tiles = q.qerl_nvfp4_tile128(codes, scales)
                if li == 0 and p == 2:
                    self.std_gate_up = (codes, scales)   # one standard copy, for comparison
                del codes, scales
                a = dev_normal((R, s.k), 0.02, gen, dev)
                b = dev_normal((s.n, R), 0.01, gen, dev)
                row.append(dict(tiles=tiles, S=S, a=a, b=b))
            self.layers.append(row)
        torch.cuda.synchronize()
        assert all(int(f.item()) == 0 for f in flags)
        self.calls = [[q.bind_linear_tiled(self.x[s.k], L["tiles"], L["S"], s.n, L["a"], L["b"],
                                           cfg.lora_scale, self.z[p][li], self.ws[p], self.y[p])
                       for p, (s, L) in enumerate(zip(self.shapes, row))]
                      for li, row in enumerate(self.layers)]
        s = self.shapes[2]
        self.gate_up_prepared = [q.bind_linear_tiled_prepared(M, row[2]["tiles"], row[2]["S"], s.n,
                                                              s.k, row[2]["b"], self.y[2],
                                                              self.ws[2]) for row in self.layers]
        self.gate_up_std = q.bind_linear_prepared(M, *self.std_gate_up, self.layers[0][2]["S"],
                                                  s.k, self.layers[0][2]["b"], self.y[2],
                                                  q.workspace(M, s.n, s.k, R, dev))
        # The gate/up call of one layer per step runs as its two halves, with
        # HIP events around the contraction half: the dominant kernel timed
        # live inside the timed steps (the same work as the whole call).
        self.probe = cfg.n_layers // 2
        L = self.layers[self.probe][2]
        self.probe_prepare = q.bind_linear_prepare(self.x[s.k], s.n, L["a"], cfg.lora_scale,
                                                   self.z[2][self.probe], self.ws[2])
        self.probe_events = []
        self.step_bytes = cfg.n_layers * sum(linear_bytes(M, s.n, s.k, R) for s in self.shapes)
        self.step_flops = cfg.n_layers * sum(linear_flops(M, s.n, s.k, R) for s in self.shapes)
        self.weight_bytes = cfg.n_layers * sum(0.5625 * s.n * s.k for s in self.shapes)

    def step(self, i, probe=False):
        import torch
        q, nl = self.q, self.cfg.n_layers
        for p, s in enumerate(self.shapes):
            q.qerl_aqn_sample_batch(4000, 0, 256 * i + p, 4, nl, self.sigma, s.k, out=self.z[p])
        for li, row in enumerate(self.calls):
            for p, call in enumerate(row):
                if probe and li == self.probe and p == 2:
                    self.probe_prepare()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    self.gate_up_prepared[li]()
                    e1.record()
                    self.probe_events.append((e0, e1))
                else:
                    call()

    def gate_up_contraction(self, li):
        """The gate/up contraction of layer li from the prepared workspace."""
        self.gate_up_prepared[li]()

    def prepare_gate_up(self):
        s, L = self.shapes[2], self.layers[0][2]
        self.q.qerl_aqn_sample(4000, 0, 2, self.sigma, s.k, out=self.z[2][0])
        for ws in (self.ws[2], self.gate_up_std.keep[-1]):
            self.q.qerl_linear_prepare(self.x[s.k], s.n, L["a"], self.cfg.lora_scale,
                                       self.z[2][0], ws)


def run_sweep(q, args, dev, stream):
    import torch
    from workloads import CONFIGS
    cfg = CONFIGS["decode_32b_sweep"]
    t_setup = time.perf_counter()
    sw = Sweep32(q, cfg, dev, keep_host_layer0=not args.no_cpu)
    t_setup = time.perf_counter() - t_setup
    for i in range(args.warmup):
        sw.step(i)
    torch.cuda.synchronize()
    clk0 = gpu_clock()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        sw.step(args.warmup + i, probe=True)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk1 = gpu_clock()
    step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    st = stats_ms(step_ms)
    med_s = st["median_ms"] / 1e3
    # the dominant kernel inside the timed steps: one gate/up contraction per step
    live = stats_ms([a.elapsed_time(b) for a, b in sw.probe_events])

    # the dominant kernel alone: the gate/up contraction (55296 x 5120, 128
    # tokens, r = 64), rotating over the 64 layers' weights
    sw.prepare_gate_up()
    s = cfg.layers[2]
    kt = batch_times(lambda i: sw.gate_up_contraction(i % cfg.n_layers), stream,
                     batches=max(10, args.steps // 10), per_batch=16)
    ks = stats_ms(kt)
    avg_s = live["mean_ms"] / 1e3
    kflops = main_kernel_flops(cfg.m, s.n, s.k, cfg.r)
    kbytes = main_kernel_bytes(cfg.m, s.n, s.k, cfg.r)
    # the same contraction on the standard (row-major) layout of one layer
    std = stats_ms(batch_times(lambda i: sw.gate_up_std(), stream, batches=5, per_batch=10))
    digest = source_digest(*M128_SOURCES)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4900)
    lib_ms = library_bf16_gemm_ms(cfg.m, s.n, s.k, dev, stream, gen, iters=50)
    roofline = {"bound": "mfma", "achieved": round(kflops / avg_s / 1e12, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kflops / avg_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("decode_gate_up_32b_m128", digest),
                "kernel": "decode_m128 (tiled weight): gate/up contraction of the 32B sweep "
                          "(55296x5120, M=128, r=64), qerl_linear_decode_tiled_prepared",
                "standard_layout_median_us": round(std["median_ms"] * 1e3, 2),
                "avg_launch_us": round(avg_s * 1e6, 2),
                "median_launch_us": round(live["median_ms"] * 1e3, 2),
                "p10_launch_us": round(live["p10_ms"] * 1e3, 2),
                "p90_launch_us": round(live["p90_ms"] * 1e3, 2),
                "timing": f"HIP events around the gate/up contraction of layer {sw.probe} in each "
                          f"of the {args.steps} timed steps (the layer's call runs as its two "
                          "halves there); avg = mean",
                "isolated_back_to_back_avg_us": round(ks["mean_ms"] * 1e3, 2),
                "isolated_note": "the same contraction launched back to back in batches of 16 "
                                 "after the steps; sustained MFMA load alone lowers the clock",
                "flops_per_launch": kflops, "bytes_per_launch": kbytes,
                "GB_per_s": round(kbytes / avg_s / 1e9, 1),
                "hbm_frac": round(kbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4),
                "roofline_us": round(max(kflops / BF16_PEAK_TFLOPS / 1e6,
                                         kbytes / HBM_PEAK_GBS / 1e3), 2),
                "library_bf16_gemm_us": round(lib_ms * 1e3, 2),
                "library_bf16_gemm_note": "reference: torch.matmul (hipBLASLt) of the same "
                                          "128 x 55296 x 5120 product with a dense bf16 weight "
                                          "(4x the weight bytes, no LoRA), random data, same box"}
    roof_step_ms = max(sw.step_flops / BF16_PEAK_TFLOPS / 1e9, sw.step_bytes / HBM_PEAK_GBS / 1e6)
    head = {
        "value": round(sw.step_bytes / med_s / 1e9, 1),
        "ms_per_step": st["median_ms"],
        "timing": dict(st, wall_s=round(wall, 4), clock_mhz_before=clk0, clock_mhz_after=clk1),
        "step": {"bytes": sw.step_bytes, "flops": sw.step_flops,
                 "nvfp4_weight_bytes": sw.weight_bytes, "calls": 4 * cfg.n_layers,
                 "tflops": round(sw.step_flops / med_s / 1e12, 1),
                 "hbm_frac": round(sw.step_bytes / med_s / 1e9 / HBM_PEAK_GBS, 4),
                 "roofline_ms": round(roof_step_ms, 4), "binding": "mfma",
                 "frac_of_roofline": round(roof_step_ms / st["median_ms"], 4),
                 "setup_s": round(t_setup, 1)},
        "roofline": roofline,
    }
    return head, sw


# --------------------------------------------------- 7B MLP decode (config 2)
# Noise ring of the 7B decode step: slots, steps sampled ahead, refill period.
# Slot safety: a refill at step i writes the slots of steps i + AHEAD - EVERY
# + 1 .. i + AHEAD after steps <= i - EVERY finished; the steps that may
# still read a slot are i - EVERY + 1 .. i + AHEAD - EVERY, so RING must
# exceed AHEAD + EVERY - 1.
NOISE_RING, NOISE_AHEAD, NOISE_EVERY = 12, 6, 4
assert NOISE_RING > NOISE_AHEAD + NOISE_EVERY - 1


def setup_decode7b(q, args, dev, to_dev):
    import torch
    from workloads import CONFIGS, make_layer
    cfg = CONFIGS["decode_7b_mlp"]
    M, R = cfg.m, cfg.r
    layers = []
    for i, s in enumerate(cfg.layers):
        L = make_layer(M, s.n, s.k, R, seed=1 + i, stage=cfg.stage,
                       outlier_frac=cfg.outlier_frac, call_id=i)
        ly = dict(name=s.name, n=s.n, k=s.k, L=L, x=to_dev(L.x), a=to_dev(L.a), b=to_dev(L.b))
        w = to_dev(L.w)
        ly["codes"], ly["scales"], ly["S"], ly["flag"] = q.qerl_quantize_nvfp4(w)
        del w
        layers.append(ly)
    torch.cuda.synchronize()
    assert all(int(ly["flag"].item()) == 0 for ly in layers)
    sigma = q.qerl_aqn_sigma(cfg.sigma_start, cfg.sigma_end, cfg.num_stages, cfg.stage)
    copies = max(1, args.copies)
    for ly in layers:
        ly["rot"] = [(ly["codes"], ly["scales"])] + [
            (ly["codes"].clone(), ly["scales"].clone()) for _ in range(copies - 1)]
        ly["ws"] = q.workspace(M, ly["n"], ly["k"], R, dev)
        ly["y"] = torch.empty((M, ly["n"]), dtype=torch.bfloat16, device=dev)
    return cfg, layers, sigma, copies


def make_chain(q, layers, cfg, to_dev, dev, sigma, copies):
    """The 7B weights as one chained decode feed-forward block: noisy RMSNorm
    (Eq. 10, noise of the gate/up group) -> fused gate/up layer (no noise of
    its own) -> down layer (its own noise) on SiLU(gate) * up, which its
    prepare forms from the gate/up output (qerl_linear_decode_swiglu).  The
    two noise vectors are drawn here, before any timing.  Returns (step
    function, algorithmic bytes of one step)."""
    import torch
    from workloads import norm_inputs
    M, R = cfg.m, cfg.r
    gu_l, dn_l = layers
    d_model, d_inter = gu_l["k"], dn_l["k"]
    xres_bits, wn_bits = norm_inputs(M, d_model, seed=41)
    xres, wnorm = to_dev(xres_bits), to_dev(wn_bits)
    z_gu = q.qerl_aqn_sample(41, 0, 0, sigma, d_model, device=dev)
    z_dn = q.qerl_aqn_sample(41, 0, 1, sigma, d_inter, device=dev)
    h = torch.empty((M, d_model), dtype=torch.bfloat16, device=dev)
    gu = [q.bind_linear(h, c, s, gu_l["S"], gu_l["a"], gu_l["b"], cfg.lora_scale, None,
                        gu_l["ws"], gu_l["y"]) for c, s in gu_l["rot"]]
    dn = [q.bind_linear(gu_l["y"], c, s, dn_l["S"], dn_l["a"], dn_l["b"], cfg.lora_scale, z_dn,
                        dn_l["ws"], dn_l["y"], entry="decode_swiglu") for c, s in dn_l["rot"]]

    def chain_step(i):
        q.qerl_rmsnorm_noisy(xres, wnorm, z_gu, 1e-6, out=h)
        gu[i % copies]()
        dn[i % copies]()

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


def run_decode7b(q, args, dev, stream, to_dev):
    import torch
    from workloads import make_layer
    cfg, layers, sigma, copies = setup_decode7b(q, args, dev, to_dev)
    M, R = cfg.m, cfg.r

    # The AQN noise of a forward pass does not depend on its activations, so a
    # second stream (default priority) samples the noise vectors a few steps
    # ahead into a ring of slots, and each step waits only for its own slot.
    # Every NOISE_EVERY steps the main stream marks its progress and the host,
    # before refilling slots, waits for the mark of NOISE_EVERY steps earlier:
    # no slot is rewritten while a queued step may still read it.
    side = torch.cuda.Stream(device=dev)
    zring = [[torch.empty(ly["k"], dtype=torch.float32, device=dev) for ly in layers]
             for _ in range(NOISE_RING)]
    z_ready = [torch.cuda.Event() for _ in range(NOISE_RING)]
    marks = {}
    calls = [[[q.bind_linear(ly["x"], c, s, ly["S"], ly["a"], ly["b"], cfg.lora_scale,
                             zring[sl][li], ly["ws"], ly["y"]) for (c, s) in ly["rot"]]
              for li, ly in enumerate(layers)] for sl in range(NOISE_RING)]

    def sample(j):
        sl = j % NOISE_RING
        for li, ly in enumerate(layers):
            q.qerl_aqn_sample(ly["L"].seed, 0, 2 * j + li, sigma, ly["k"],
                              out=zring[sl][li], stream=side)
        z_ready[sl].record(side)

    def step(i):
        sl = i % NOISE_RING
        stream.wait_event(z_ready[sl])
        for li in range(len(layers)):
            calls[sl][li][i % copies]()
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
    steps = max(100, args.steps)
    st = stats_ms(event_times(step, steps, stream, warmup=max(NOISE_EVERY, args.warmup)))
    torch.cuda.synchronize()
    step_bytes = sum(linear_bytes(M, ly["n"], ly["k"], R) for ly in layers)
    out = {"workload": "decode_7b_mlp: Qwen2.5-7B-shaped MLP, M=64 (8 prompts x 8 samples), "
                       "gate/up 37888x3584 + down 3584x18944 NVFP4, LoRA r=32, AQN stage 1/10",
           "weight_copies_rotated": copies,
           "GB_per_s": round(step_bytes / (st["median_ms"] / 1e3) / 1e9, 1),
           "hbm_frac": round(step_bytes / (st["median_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "timing": st}

    # the gate/up contraction kernel alone
    ly = layers[0]
    q.qerl_linear_prepare(ly["x"], ly["n"], ly["a"], cfg.lora_scale, zring[0][0], ly["ws"])
    kcalls = [q.bind_linear_prepared(M, c, s_, ly["S"], ly["k"], ly["b"], ly["y"], ly["ws"])
              for c, s_ in ly["rot"]]
    kt = batch_times(lambda i: kcalls[i % copies](), stream, batches=10, per_batch=12)
    ks = stats_ms(kt)
    kbytes = main_kernel_bytes(M, ly["n"], ly["k"], R)
    avg_s = ks["mean_ms"] / 1e3
    out["gate_up_kernel"] = {
        "bound": "hbm", "achieved": round(kbytes / avg_s / 1e9, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(kbytes / avg_s / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic("decode_main_gate_up_7b", source_digest(*LDS_SOURCES)),
        "kernel": "decode_lds<2,5> (gate/up 37888x3584, M=64, r=32)",
        "avg_launch_us": round(avg_s * 1e6, 2),
        "median_launch_us": round(ks["median_ms"] * 1e3, 2),
        "p10_launch_us": round(ks["p10_ms"] * 1e3, 2),
        "p90_launch_us": round(ks["p90_ms"] * 1e3, 2), "bytes_per_launch": kbytes}

    # the same weights as a chained feed-forward block
    chain_step, chain_bytes = make_chain(q, layers, cfg, to_dev, dev, sigma, copies)
    cs = stats_ms(event_times(chain_step, steps, stream, warmup=args.warmup))
    out["mlp_chain"] = {
        "workload": "noisy RMSNorm -> gate/up -> down on SiLU(gate)*up (formed in the down "
                    "layer's prepare), M=64",
        "us_per_step": round(cs["median_ms"] * 1e3, 2),
        "GB_per_s": round(chain_bytes / (cs["median_ms"] / 1e3) / 1e9, 1),
        "frac_hbm": round(chain_bytes / (cs["median_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "timing": cs}

    # the gate/up weight as MXFP4 in the NVFP4 layout: general and power-of-two
    # dequantization, three interleaved rounds, median of all launches
    gl = layers[0]
    mrot, mg, mflag = make_mxfp4(q, gl, cfg, make_layer, to_dev, copies, zring[0][0])
    mx = {"workload": "gate/up 37888x3584 MXFP4 weight in the NVFP4 layout, M=64, r=32",
          "range_flag": int(mflag.item())}
    mx_t = {"general": [], "pow2": []}
    mcalls = {e: [q.bind_linear_prepared(M, c, s_, mg, gl["k"], gl["b"], gl["y"], gl["ws"],
                                         entry=e) for c, s_ in mrot]
              for e in ("decode", "decode_mxfp4")}
    for _ in range(3):
        for name, e in (("general", "decode"), ("pow2", "decode_mxfp4")):
            mx_t[name] += batch_times(lambda i: mcalls[e][i % copies](), stream, batches=4,
                                      per_batch=12)
    for name, v in mx_t.items():
        mx[name + "_us"] = round(stats_ms(v)["median_ms"] * 1e3, 2)
    mx["pow2_GB_per_s"] = round(kbytes / (mx["pow2_us"] * 1e-6) / 1e9, 1)
    out["mxfp4_decode"] = mx
    del mrot, mcalls, kcalls, layers, calls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ------------------------------------------- 7B chained decode layer (f4 row)
def run_layer7b(q, args, dev, stream, copies=4):
    """One whole Qwen2.5-7B decode layer at 64 tokens as a chain of library
    calls: noisy RMSNorm -> q/k/v [4608, 3584] -> attention over a
    one-position context (28 q / 4 kv heads of 128) -> o [3584, 3584] ->
    noisy RMSNorm -> gate/up [37888, 3584] -> SiLU(gate) * up -> down [3584,
    18944]; LoRA r=32 everywhere, AQN stage 1.  Two noise variants: one
    vector per call (q/k/v and gate/up groups in the RMSNorm scale, o and
    down in their input), and one row per token on every linear call.
    Weights (seeded, on the device) are rotated over `copies` layers (524 MB)
    so that the Infinity Cache cannot hold them."""
    import torch
    M, R, H, I, HQ, HKV, DH = 64, 32, 3584, 18944, 28, 4, 128
    shapes = [((HQ + 2 * HKV) * DH, H), (H, HQ * DH), (2 * I, H), (H, I)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7000)
    layers = []
    for c in range(copies):
        row = []
        for n, k in shapes:
            w = dev_normal((n, k), 0.02, gen, dev)
            codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
            del w
            row.append(dict(codes=codes, scales=scales, S=S, n=n, k=k,
                            a=dev_normal((R, k), 0.02, gen, dev),
                            b=dev_normal((n, R), 0.01, gen, dev)))
        layers.append(row)
    x = dev_normal((M, H), 1.0, gen, dev)
    w1 = (1.0 + 0.05 * torch.randn(H, generator=gen, device=dev)).to(torch.bfloat16)
    w2 = (1.0 + 0.05 * torch.randn(H, generator=gen, device=dev)).to(torch.bfloat16)
    sig = 1e-2
    zv = [q.qerl_aqn_sample(7000, 0, i, sig, k, device=dev) for i, (_, k) in enumerate(shapes)]
    zr = [q.qerl_aqn_sample_rows(7000, 0, i, sig, M, k, device=dev)
          for i, (_, k) in enumerate(shapes)]
    h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    att = torch.empty((M, HQ * DH), dtype=torch.bfloat16, device=dev)
    act = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    ys = [torch.empty((M, n), dtype=torch.bfloat16, device=dev) for n, _ in shapes]
    wss = [q.workspace(M, n, k, R, dev) for n, k in shapes]
    ins = [h, att, h, act]

    def bound(per_row):
        calls = []
        for row in layers:
            c = []
            for i, L in enumerate(row):
                inp = ins[i]
                entry = "decode_rownoise" if per_row else "decode"
                z = zr[i] if per_row else (zv[i] if i in (1, 3) else None)
                if i == 3 and not per_row:
                    inp, entry = ys[2], "decode_swiglu"
                c.append(q.bind_linear(inp, L["codes"], L["scales"], L["S"], L["a"], L["b"], 2.0,
                                       z, wss[i], ys[i], entry=entry))
            calls.append(c)
        return calls

    shared, rows = bound(False), bound(True)

    def step_shared(i):
        c = shared[i % copies]
        q.qerl_rmsnorm_noisy(x, w1, zv[0], 1e-6, out=h)
        c[0]()
        q.qerl_attention_stub(ys[0], HQ, HKV, DH, out=att)
        c[1]()
        q.qerl_rmsnorm_noisy(ys[1], w2, zv[2], 1e-6, out=h)
        c[2]()
        c[3]()

    def step_rows(i):
        c = rows[i % copies]
        q.qerl_rmsnorm_noisy(x, w1, None, 1e-6, out=h)
        c[0]()
        q.qerl_attention_stub(ys[0], HQ, HKV, DH, out=att)
        c[1]()
        q.qerl_rmsnorm_noisy(ys[1], w2, None, 1e-6, out=h)
        c[2]()
        q.qerl_swiglu(ys[2], out=act)
        c[3]()

    # algorithmic bytes of a layer: the linear calls without their noise
    # input, the RMSNorms (x in, y out, w), the stub (v heads in, heads out)
    lin = sum(linear_bytes(M, n, k, R) - 4 * k for n, k in shapes)
    base = lin + 2 * (4 * M * H + 2 * H) + 2 * M * (HKV + HQ) * DH
    # per call: z of the two RMSNorms, o and down; down reads gate and up
    shared_bytes = base + 4 * (H + H + H + I) + 2 * M * I
    # per row: z rows of the four linear calls; the SwiGLU kernel in between
    rows_bytes = base + 4 * M * (3 * H + I) + 6 * M * I
    out = {"workload": "Qwen2.5-7B decode layer at M=64: noisy RMSNorm, q/k/v, attention stub "
                       "(one-position context), o, noisy RMSNorm, gate/up, SiLU*up, down; "
                       f"LoRA r=32, AQN stage 1; weights rotated over {copies} layers"}
    for name, fn, nbytes in (("per_call_noise", step_shared, shared_bytes),
                             ("per_row_noise", step_rows, rows_bytes)):
        st = stats_ms(event_times(fn, max(100, args.steps), stream, warmup=args.warmup))
        out[name] = {"us_per_layer": round(st["median_ms"] * 1e3, 2),
                     "GB_per_s": round(nbytes / (st["median_ms"] / 1e3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (st["median_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "timing": st}
    del layers, shared, rows
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------- 7B prefill + backward (config 3)
def run_prefill7b(q, args, dev, stream, to_dev):
    import torch
    from workloads import CONFIGS, make_layer, normal_bf16
    pc = CONFIGS["prefill_7b"]
    psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
    reps = 20
    per_layer, t_full, t_main, pflops = [], 0.0, 0.0, 0.0
    for i, s in enumerate(pc.layers):
        L = make_layer(pc.m, s.n, s.k, pc.r, seed=11 + i, stage=pc.stage, call_id=i)
        x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
        codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
        del w
        z = q.qerl_aqn_sample(L.seed, 0, i, psig, s.k, device=dev)
        ws = q.workspace(pc.m, s.n, s.k, pc.r, dev)
        y = torch.empty((pc.m, s.n), dtype=torch.bfloat16, device=dev)
        full = q.bind_linear(x, codes, scales, S, a, b, pc.lora_scale, z, ws, y, entry="prefill")
        tf = stats_ms(event_times(lambda i: full(), reps, stream))
        q.qerl_linear_prepare(x, s.n, a, pc.lora_scale, z, ws)
        tm = stats_ms(event_times(lambda i: q.qerl_linear_prefill_prepared(
            pc.m, codes, scales, S, s.k, b, y, ws), reps, stream))
        fl = linear_flops(pc.m, s.n, s.k, pc.r)
        per_layer.append({"layer": f"{s.name} {s.n}x{s.k}",
                          "tflops": round(fl / tf["median_ms"] / 1e9, 1),
                          "gemm_tflops": round(fl / tm["median_ms"] / 1e9, 1),
                          "ms": tf["median_ms"], "gemm_ms": tm["median_ms"],
                          "p10_ms": tf["p10_ms"], "p90_ms": tf["p90_ms"]})
        t_full += tf["median_ms"]
        t_main += tm["median_ms"]
        pflops += fl
        del x, a, b, codes, scales, ws, y, full
    out = {"workload": "prefill_7b (qkv 4608x3584 + down 3584x18944, M=4096, r=32, AQN stage "
                       "5/10)",
           "tflops": round(pflops / t_full / 1e9, 1), "gemm_tflops": round(pflops / t_main / 1e9, 1),
           "ms": round(t_full, 4),
           "frac_bf16_peak": round(pflops / t_full / 1e9 / BF16_PEAK_TFLOPS, 4),
           "gemm_frac_bf16_peak": round(pflops / t_main / 1e9 / BF16_PEAK_TFLOPS, 4),
           "reps": reps, "layers": per_layer}

    # backward through the frozen NVFP4 weight of the 7B down layer, 4096 tokens
    s_dn = pc.layers[1]
    L = make_layer(pc.m, s_dn.n, s_dn.k, pc.r, seed=12, stage=pc.stage, call_id=1)
    x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
    codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
    del w
    z = q.qerl_aqn_sample(L.seed, 0, 1, psig, s_dn.k, device=dev)
    dy = to_dev(normal_bf16((pc.m, s_dn.n), 1.0, 12050))
    bws = torch.empty(q.lib.qerl_linear_backward_workspace_bytes(pc.m, s_dn.n, s_dn.k, pc.r),
                      dtype=torch.uint8, device=dev)
    tb = stats_ms(event_times(lambda i: q.qerl_linear_backward(dy, x, codes, scales, S, a, b,
                                                               pc.lora_scale, z, workspace=bws),
                              reps, stream))
    mm, nn, kk, rr = pc.m, s_dn.n, s_dn.k, pc.r
    bflops = (2.0 * mm * nn * kk          # dy W_hat
              + 2.0 * mm * rr * kk * 3     # t = x_t A^T, gs A, dA
              + 2.0 * mm * nn * rr * 2)    # gs = dy B, dB
    out["backward"] = {"workload": f"backward of the 7B down layer: dy {mm}x{nn}, W {nn}x{kk} "
                                   f"NVFP4, r={rr} (dx, dA, dB)",
                       "ms": tb["median_ms"], "p10_ms": tb["p10_ms"], "p90_ms": tb["p90_ms"],
                       "tflops": round(bflops / tb["median_ms"] / 1e9, 1),
                       "frac_bf16_peak": round(bflops / tb["median_ms"] / 1e9 / BF16_PEAK_TFLOPS,
                                               4)}
    del x, a, b, codes, scales, dy, bws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ------------------------------------ 14B bulk quantizer + prefill (config 5)
class Model14b:
    """Every linear weight of a Qwen2.5-14B-shaped model (48 layers x {q, k,
    v, o, gate, up, down}) as bf16 on the device (seeded), with the output
    buffers of the bulk quantization and one bound quantize call each."""

    def __init__(self, q, cfg, dev):
        import torch
        gen = torch.Generator(device=dev)
        gen.manual_seed(5000)
        self.cfg = cfg
        self.tensors = []
        for li in range(cfg.n_layers):
            for s in cfg.layers:
                w = dev_normal((s.n, s.k), 0.02, gen, dev)
                codes = torch.empty((s.n, s.k // 2), dtype=torch.uint8, device=dev)
                scales = torch.empty((s.n, s.k // 16), dtype=torch.uint8, device=dev)
                S = torch.empty(1, dtype=torch.float32, device=dev)
                flag = torch.empty(1, dtype=torch.int32, device=dev)
                self.tensors.append(dict(layer=li, name=s.name, n=s.n, k=s.k, w=w, codes=codes,
                                         scales=scales, S=S, flag=flag))
        self.calls = [q.bind_quantize_nvfp4(t["w"], t["codes"], t["scales"], t["S"], t["flag"])
                      for t in self.tensors]
        self.batch = q.bind_quantize_nvfp4_batch(
            [t["w"] for t in self.tensors],
            [(t["codes"], t["scales"], t["S"], t["flag"]) for t in self.tensors])
        self.elements = sum(t["n"] * t["k"] for t in self.tensors)

    def quantize_all(self, i=0):
        """The bulk quantization: one batched call over every tensor."""
        self.batch()

    def quantize_each(self, i=0):
        """The same tensors with one qerl_quantize_nvfp4 call each."""
        for c in self.calls:
            c()


def run_14b(q, args, dev, stream):
    import torch
    from workloads import CONFIGS
    cfg = CONFIGS["quantize_prefill_14b"]
    mdl = Model14b(q, cfg, dev)
    torch.cuda.synchronize()
    qt = stats_ms(event_times(mdl.quantize_all, 5, stream, warmup=1))
    flags = torch.stack([t["flag"] for t in mdl.tensors])
    assert int(flags.max().item()) == 0
    qe = stats_ms(event_times(mdl.quantize_each, 5, stream, warmup=1))
    qbytes = 2.5625 * mdl.elements
    out = {"workload": "quantize_prefill_14b: bulk NVFP4 quantization of every linear weight of a "
                       "Qwen2.5-14B-shaped model (48 layers x q, k, v, o, gate, up, down; "
                       "N(0, 0.02^2) bf16), then prefill M=16384 through layer 0's o, gate, up "
                       "and down (r=32, AQN stage 1)",
           "quantizer": {"tensors": len(mdl.tensors), "elements": mdl.elements,
                         "bytes_per_elem": 2.5625, "ms": qt["median_ms"],
                         "GB_per_s": round(qbytes / qt["median_ms"] / 1e6, 1),
                         "hbm_frac": round(qbytes / qt["median_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                         "roofline_ms": round(qbytes / HBM_PEAK_GBS / 1e6, 4), "timing": qt,
                         "entry": "qerl_quantize_nvfp4_batch (one call, count + 2 launches)",
                         "per_tensor_calls_ms": qe["median_ms"]}}
    # prefill through layer 0's o, gate, up, down at 16384 tokens
    M, R = cfg.m, cfg.r
    sig = q.qerl_aqn_sigma(cfg.sigma_start, cfg.sigma_end, cfg.num_stages, cfg.stage)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5100)
    xs = {}
    lib_gen = torch.Generator(device=dev)
    lib_gen.manual_seed(5200)
    per_layer, t_tot, f_tot, lib_tot, lib_fl = [], 0.0, 0.0, 0.0, 0.0
    layer0 = {t["name"]: t for t in mdl.tensors if t["layer"] == 0}
    mdl.calls = None
    mdl.tensors = None
    for t in layer0.values():
        del t["w"]
    torch.cuda.empty_cache()
    for name in ("o", "gate", "up", "down"):
        t = layer0[name]
        n, k = t["n"], t["k"]
        if k not in xs:
            xs[k] = dev_normal((M, k), 1.0, gen, dev)
        a = dev_normal((R, k), 0.02, gen, dev)
        b = dev_normal((n, R), 0.01, gen, dev)
        z = q.qerl_aqn_sample(5100, 0, len(per_layer), sig, k, device=dev)
        ws = q.workspace(M, n, k, R, dev)
        y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        call = q.bind_linear(xs[k], t["codes"], t["scales"], t["S"], a, b, cfg.lora_scale, z, ws,
                             y, entry="prefill")
        tt = stats_ms(event_times(lambda i: call(), 20, stream))
        fl = linear_flops(M, n, k, R)
        del a, b, z, ws, y, call
        lib_ms = library_bf16_gemm_ms(M, n, k, dev, stream, lib_gen)
        per_layer.append({"layer": f"{name} {n}x{k}", "ms": tt["median_ms"],
                          "p10_ms": tt["p10_ms"], "p90_ms": tt["p90_ms"],
                          "tflops": round(fl / tt["median_ms"] / 1e9, 1),
                          "library_bf16_gemm_ms": lib_ms,
                          "library_bf16_gemm_tflops": round(2.0 * M * n * k / lib_ms / 1e9, 1)})
        t_tot += tt["median_ms"]
        f_tot += fl
        lib_tot += lib_ms
        lib_fl += 2.0 * M * n * k
    out["prefill"] = {"tokens": M, "ms": round(t_tot, 4), "tflops": round(f_tot / t_tot / 1e9, 1),
                      "frac_bf16_peak": round(f_tot / t_tot / 1e9 / BF16_PEAK_TFLOPS, 4),
                      "roofline_ms": round(f_tot / BF16_PEAK_TFLOPS / 1e9, 4),
                      "library_bf16_gemm_tflops": round(lib_fl / lib_tot / 1e9, 1),
                      "library_bf16_gemm_note": "reference: torch.matmul (hipBLASLt) of the same "
                                                "four products with dense bf16 weights (no "
                                                "dequantization, no LoRA), random data, same box",
                      "layers": per_layer}
    del mdl, xs, layer0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------- noisy RMSNorm
def run_rmsnorm(q, dev, stream, to_dev):
    import torch
    from workloads import norm_inputs
    res = []
    for m, d, copies_n in ((4096, 3584, 10), (64, 3584, 1)):
        xs_, ws_ = norm_inputs(m, d, seed=31)
        wd = to_dev(ws_)
        xcopies = [to_dev(xs_) for _ in range(copies_n)]
        ycopies = [torch.empty_like(xcopies[0]) for _ in range(copies_n)]
        zd = q.qerl_aqn_sample(31, 0, 0, 1e-2, d, device=dev)
        st = stats_ms(event_times(lambda i: q.qerl_rmsnorm_noisy(
            xcopies[i % copies_n], wd, zd, 1e-6, out=ycopies[i % copies_n]), 100, stream,
            warmup=5))
        t = st["median_ms"] / 1e3
        nbytes = 4 * m * d + 2 * d + 4 * d
        res.append({"workload": f"noisy RMSNorm {m}x{d} (Qwen2.5-7B hidden)",
                    "us": round(t * 1e6, 2), "GB_per_s": round(nbytes / t / 1e9, 1),
                    "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes})
    return res


# --------------------------------------------------------- oracle on the host
def oracle_sweep_rate(sw, min_seconds=12.0, max_reps=100):
    """The oracle running a labelled slice of the headline step on the host:
    layer 0 of the 32B sweep, the first 512 output rows of each of its four
    projections, all 128 tokens and all K: per projection, draw the noise
    vector, dequantize the NVFP4 weight slice and evaluate the fp64 linear
    layer with the LoRA branch.  The weight slices are quantized by the oracle
    before timing (the GPU step also runs on weights quantized beforehand)."""
    import numpy as np
    import threadpoolctl
    import torch
    from oracle import aqn, linear, nvfp4
    cfg = sw.cfg
    rows = 512
    prepared = []
    for p, s in enumerate(sw.shapes):
        codes, scales, S = nvfp4.quantize(sw.host_w0[p])
        L = sw.layers[0][p]
        host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        prepared.append((s, codes, scales, S, host(sw.x[s.k]), host(L["a"]),
                         host(L["b"][:rows])))
    sbytes = sum(linear_bytes(cfg.m, rows, s.k, cfg.r) for s in sw.shapes)
    reps, t0 = 0, time.perf_counter()
    while True:
        for p, (s, codes, scales, S, x, a, b) in enumerate(prepared):
            z = aqn.sample(4000, 0, 256 * reps + p, sw.sigma, s.k)
            w_hat = nvfp4.dequantize(codes, scales, S)
            linear.linear(x, w_hat, z, a, b, cfg.lora_scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
            if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    return {"value": round(reps * sbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} repetition(s) in {dt:.1f} s of a slice of the 32B sweep step: "
                      f"layer 0, the first {rows} output rows of each of qkv, o, gate/up and "
                      "down (all 128 tokens, all K, r=64): noise vector, NVFP4 dequantization, "
                      f"fp64 linear with LoRA; {sbytes / 1e6:.1f} MB algorithmic per repetition; "
                      "weights quantized by the oracle before timing; noise and dequantization "
                      f"on one thread, the fp64 matmuls on {threads} BLAS threads of "
                      f"{len(os.sched_getaffinity(0))} host cores"}


# ------------------------------------------------------------ profiling passes
def profile_pass(q, args, dev, stream, to_dev):
    import torch
    from workloads import CONFIGS, make_layer, normal_bf16
    kind = args.profile
    if kind in ("decode", "sweep32", "rmsnorm", "backward", "quant14b"):
        calibration_copy(dev)
    if kind == "sweep32":
        sw = Sweep32(q, CONFIGS["decode_32b_sweep"], dev)
        for i in range(3):
            sw.step(i)
        sw.prepare_gate_up()
        for i in range(PROFILE_LAUNCHES):
            sw.gate_up_contraction(i % sw.cfg.n_layers)
        torch.cuda.synchronize()
        print(f"profile pass done: copy {COPY_BYTES} B, 3 sweep steps, {PROFILE_LAUNCHES} 32B "
              "gate/up contractions at M=128")
        return
    if kind == "quant14b":
        mdl = Model14b(q, CONFIGS["quantize_prefill_14b"], dev)
        mdl.quantize_all()
        torch.cuda.synchronize()
        print(f"profile pass done: copy {COPY_BYTES} B, one bulk quantization of "
              f"{len(mdl.tensors)} tensors")
        return
    if kind in ("prefill", "prefill14b"):
        if kind == "prefill":
            pc = CONFIGS["prefill_7b"]
            shapes = pc.layers
        else:
            pc = CONFIGS["quantize_prefill_14b"]
            shapes = [s for s in pc.layers if s.name in ("o", "gate", "up", "down")]
        psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
        gen = torch.Generator(device=dev)
        gen.manual_seed(5200)
        for i, s in enumerate(shapes):
            x = dev_normal((pc.m, s.k), 1.0, gen, dev)
            w = dev_normal((s.n, s.k), 0.02, gen, dev)
            a = dev_normal((pc.r, s.k), 0.02, gen, dev)
            b = dev_normal((s.n, pc.r), 0.01, gen, dev)
            codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
            del w
            z = q.qerl_aqn_sample(5200, 0, i, psig, s.k, device=dev)
            ws = q.workspace(pc.m, s.n, s.k, pc.r, dev)
            y = torch.empty((pc.m, s.n), dtype=torch.bfloat16, device=dev)
            q.qerl_linear_prepare(x, s.n, a, pc.lora_scale, z, ws)
            for _ in range(3):
                q.qerl_linear_prefill_prepared(pc.m, codes, scales, S, s.k, b, y, ws)
            torch.cuda.synchronize()
            del x, a, b, codes, scales, ws, y
        print(f"profile pass done: {kind}, one prepare and 3 GEMMs per layer")
        return
    if kind == "rmsnorm":
        from workloads import norm_inputs
        m, d, copies, launches = 4096, 3584, 10, 20
        x, w = norm_inputs(m, d, seed=31)
        wd = to_dev(w)
        xs = [to_dev(x) for _ in range(copies)]
        ys = [torch.empty_like(xs[0]) for _ in range(copies)]
        z = q.qerl_aqn_sample(31, 0, 0, 1e-2, d, device=dev)
        for i in range(launches):
            q.qerl_rmsnorm_noisy(xs[i % copies], wd, z, 1e-6, out=ys[i % copies])
        torch.cuda.synchronize()
        print(f"profile pass done: copy {COPY_BYTES} B, {launches} noisy RMSNorms {m}x{d}")
        return
    if kind == "backward":
        pc = CONFIGS["prefill_7b"]
        s_dn = pc.layers[1]
        L = make_layer(pc.m, s_dn.n, s_dn.k, pc.r, seed=12, stage=pc.stage, call_id=1)
        x, w, a, b = to_dev(L.x), to_dev(L.w), to_dev(L.a), to_dev(L.b)
        codes, scales, S, _ = q.qerl_quantize_nvfp4(w)
        del w
        psig = q.qerl_aqn_sigma(pc.sigma_start, pc.sigma_end, pc.num_stages, pc.stage)
        z = q.qerl_aqn_sample(L.seed, 0, 1, psig, s_dn.k, device=dev)
        dy = to_dev(normal_bf16((pc.m, s_dn.n), 1.0, 12050))
        for _ in range(3):
            q.qerl_linear_backward(dy, x, codes, scales, S, a, b, pc.lora_scale, z)
        torch.cuda.synchronize()
        print(f"profile pass done: 3 backward calls of the 7B down layer at M={pc.m}")
        return
    # decode / chain / mxfp4: the 7B MLP weights
    cfg, layers, sigma, copies = setup_decode7b(q, args, dev, to_dev)
    M = cfg.m
    if kind == "chain":
        chain_step, _ = make_chain(q, layers, cfg, to_dev, dev, sigma, copies)
        for i in range(PROFILE_LAUNCHES):
            chain_step(i)
        torch.cuda.synchronize()
        print(f"profile pass done: {PROFILE_LAUNCHES} chained decode feed-forward steps")
        return
    gl = layers[0]
    z = q.qerl_aqn_sample(gl["L"].seed, 0, 0, sigma, gl["k"], device=dev)
    if kind == "mxfp4":
        mrot, mg, _ = make_mxfp4(q, gl, cfg, make_layer, to_dev, copies, z)
        for fn in (q.qerl_linear_decode_prepared, q.qerl_linear_decode_prepared_mxfp4):
            for i in range(PROFILE_LAUNCHES):
                fn(M, *mrot[i % copies], mg, gl["k"], gl["b"], gl["y"], gl["ws"])
        torch.cuda.synchronize()
        print(f"profile pass done: {PROFILE_LAUNCHES} MXFP4 gate/up contractions with each "
              "dequantization")
        return
    q.qerl_linear_prepare(gl["x"], gl["n"], gl["a"], cfg.lora_scale, z, gl["ws"])
    for i in range(PROFILE_LAUNCHES):
        c, s = gl["rot"][i % copies]
        q.qerl_linear_decode_prepared(M, c, s, gl["S"], gl["k"], gl["b"], gl["y"], gl["ws"])
    torch.cuda.synchronize()
    print(f"profile pass done: copy {COPY_BYTES} B, {PROFILE_LAUNCHES} gate/up contractions "
          f"({main_kernel_bytes(M, gl['n'], gl['k'], cfg.r):.0f} algorithmic B each)")


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

    dev = "cuda:0"
    torch.cuda.set_device(0)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    stream = torch.cuda.current_stream()

    if args.profile:
        profile_pass(q, args, dev, stream, to_dev)
        return

    parts = set(args.only or PARTS)
    out = {"metric": "NVFP4+LoRA linear: decode weight-stream GB/s and prefill TFLOP/s, "
                     "% roofline",
           "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (NVFP4 weights)",
           "data": "synthetic",
           "config": {"workload": "decode_32b_sweep: Qwen2.5-32B-shaped decode step, 64 layers x "
                                  "{qkv 7168x5120, o 5120x5120, gate/up 55296x5120, down "
                                  "5120x27648} NVFP4 (17.55 GB streamed per step), M=128 (8 "
                                  "prompts x 16 samples), LoRA r=64 on every projection, AQN "
                                  "stage 1/10 with one noise vector per projection and layer; "
                                  "weights held in the tiled NVFP4 layout",
                      "global_batch": 128, "parallelism": "none (1 GPU)"}}
    cpu = None
    if "sweep" in parts:
        head, sw = run_sweep(q, args, dev, stream)
        out["value"] = head["value"]
        out["ms_per_step"] = head["ms_per_step"]
        out["roofline"] = head["roofline"]
        out["timing"] = head["timing"]
        out["step"] = head["step"]
        if not args.no_cpu:
            cpu = oracle_sweep_rate(sw)
        del sw
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if "decode7b" in parts:
        out["decode_7b_mlp"] = run_decode7b(q, args, dev, stream, to_dev)
    if "layer7b" in parts:
        out["decode_layer_7b"] = run_layer7b(q, args, dev, stream)
    if "prefill7b" in parts:
        out["prefill_7b"] = run_prefill7b(q, args, dev, stream, to_dev)
    if "q14b" in parts:
        out["quantize_prefill_14b"] = run_14b(q, args, dev, stream)
    if "rmsnorm" in parts:
        out["rmsnorm"] = run_rmsnorm(q, dev, stream, to_dev)
    out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
