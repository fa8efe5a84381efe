"""Build libkivi.so (HIP kernels for gfx950 + the C-ABI front end) in-tree.

    python -m kv_cache_quantization_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkivi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: the quantizer's subtract / divide / round must be the
# separate IEEE operations the definition states; FMAs are written explicitly
# where the decode path wants them.  Packed fp32 instructions are disabled.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wno-inline-asm",
    "-I", os.path.join(ROOT, "include"),
]
# MFMA results in VGPRs rather than AGPRs: the decode loop also touches its
# accumulators with vector ALU code, and an AGPR home costs a copy in and out
# per group (and the registers of a fourth wave per SIMD).
DEVICE = [
    "--offload-arch=gfx950", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    extra_all = tuple(extra)
    units = [("kivi_kernels.hip", DEVICE), ("kivi_api.cpp", ["-D__HIP_PLATFORM_AMD__"])]
    for src, extra in units:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + COMMON + extra + (list(extra_all) if src.endswith(".hip") else []) + \
            ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
