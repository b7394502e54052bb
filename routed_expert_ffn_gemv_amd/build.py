"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libmoe.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 ops are switched off for all device code.  Code object v5:
# the HIP runtime bundled with PyTorch loads v5 (not v6) code objects.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


HOST_ONLY = {"host_tier.cpp"}
# Per-file device flags.  The fused decode layer kernel is built with the
# ILP-first machine scheduler: measured 19.9 -> 19.0 us per one-token layer,
# unchanged for four tokens.
FILE_FLAGS = {"layer.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        # .hip: device and host code; host_tier.cpp: plain C++ (the CPU
        # tier, no device pass); other .cpp: host code that calls HIP
        name = os.path.basename(src)
        lang = ["-x", "hip"] if src.endswith(".hip") else (["-x", "c++"] if name in HOST_ONLY else [])
        cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(name, []) + lang + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            noise = "not a recognized feature for this target"
            msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
            if msg.strip():
                print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
