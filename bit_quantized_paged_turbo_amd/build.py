"""Build libxq.so (the C ABI plus the gfx950 kernels) in-tree with hipcc.

    python -m bit_quantized_paged_turbo_amd.build [--asm]

Every HIP source is compiled with packed-FP32 instructions disabled; the codec
(quantize_append.hip) also forbids FP contraction itself so its codes are bit-exact.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libxq.so")
ARCH = "gfx950"

SOURCES = ["xq_abi.cpp", "quantize_append.hip", "decode_attention.hip", "prefill_attention.hip", "hbm_probe.hip"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
               "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
               *DEVICE_FLAGS, "-c", path, "-o", obj]
        if asm:
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libxq.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(asm="--asm" in sys.argv, verbose=True))
