"""Build the Sol-Attn HIP library for gfx950 in-tree (libsolattn.so next to
this file).  Usage: python -m block_sparse_video_solattn_amd.build"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsolattn.so")
SOURCES = ["solattn_api.cpp", "pool.hip", "route.hip", "attn_bf16.hip", "attn_f32.hip", "probe.hip",
           "transport.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 instructions stay off (plain fp32 VALU only)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in arch VGPRs: the online-softmax rescale touches
        # the output accumulator with VALU ops, and AGPR-resident accumulators
        # made the compiler copy all of them to VGPRs on every loop iteration
        "-mllvm", "-amdgpu-mfma-vgpr-form=true",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libsolattn.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-o", tmp, "-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout)
        raise RuntimeError("hipcc failed building %s" % LIB)
    if verbose and res.stdout.strip():
        print(res.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
