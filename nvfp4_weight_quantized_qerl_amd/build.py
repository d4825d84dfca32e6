"""Build libqerl.so (all HIP sources, gfx950) in-tree with hipcc.

    python nvfp4_weight_quantized_qerl_amd/build.py

Every source under csrc/ is compiled to an object under _build/ (in
parallel), then linked into nvfp4_weight_quantized_qerl_amd/libqerl.so.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqerl.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU forms are kept out of all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Exact arithmetic is part of the contract: no contraction, no flushing.
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # Per-kernel resource report, checked below for scratch use.
    "-Rpass-analysis=kernel-resource-usage",
]

# Kernels allowed to use scratch memory, with the bytes per lane they may
# use: the 256 x 256 prefill tile keeps one 8-byte value there across its K
# loop.  Any other kernel with scratch fails the build (a spill inside a hot
# loop costs far more than any change that causes it could gain).
SCRATCH_ALLOWED = {"_ZN4qerl7prefill4gemmILi2ELi4ELi128ELi64ELi2EEEvNS0_4ArgsE": 12}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _scratch_users(text):
    """(kernel, bytes per lane) of every kernel whose resource report shows
    scratch, from hipcc's kernel-resource-usage remarks."""
    out, name = [], None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line and name:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size > 0:
                out.append((name, size))
    return out


def _compile(src, verbose):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = res.stdout + res.stderr
    msgs = "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msgs}")
    bad = [(k, b) for k, b in _scratch_users(text) if b > SCRATCH_ALLOWED.get(k, 0)]
    if bad:
        raise RuntimeError(f"{src}: kernels using scratch memory: {bad}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose=False, jobs=None):
    """Compile every HIP source and link libqerl.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
