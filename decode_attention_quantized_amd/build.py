"""Build libkvq.so in-tree with hipcc for gfx950.

    python decode_attention_quantized_amd/build.py

The HIP sources are compiled with packed-FP32 instructions disabled and with IEEE fp32
division/rounding (no fast-math): the quantizer must match a correctly rounded reference
bit for bit.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
# MFMA results stay in ordinary VGPRs: with AGPRs available (one wave per SIMD) the compiler would
# otherwise copy the accumulators between the two register files around every VALU update.
# Leading scalar kernel arguments are preloaded into SGPRs at wave launch (the decode kernels put
# what their first memory requests need first), which saves the argument-block round trip.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("build failed: " + " ".join(cmd))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src, dev in [("kvq_kernels.hip", True), ("kvq_api.cpp", False)]:
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC] + COMMON + (DEVICE if dev else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
