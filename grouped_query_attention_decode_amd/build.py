"""Build libgqa.so in-tree with hipcc for gfx950.

    python -m grouped_query_attention_decode_amd.build

Compiles every source under ``csrc/`` into one shared library next to this
file.  Each call compiles from scratch (a few tens of seconds).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libgqa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gqa_kernels.hip", "gqa_api.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 ALU ops.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Kernel source only: matrix-core (MFMA) accumulators in ordinary VGPRs.  The
# default places a loop-carried accumulator in AGPRs and copies it to VGPRs
# and back every tile (the 32 x 32 kernel at one wave per SIMD: ~470 AGPR
# reads and ~600 writes per kernel, most in its tile loop; ~20 with this
# form).  Measured, same bits: sweep G = 1 46.3 -> 44.5 us, MQA 56.8 -> 56.6,
# the other workloads unchanged.
#
# -amdgpu-kernarg-preload-count=3: the decode kernels take seq_lens, B and T
# as their first three arguments, and the command processor places them in
# scalar registers at dispatch, so the lengths' load goes out without first
# waiting for the argument block to load (a code object prologue loads them
# where the firmware does not preload).  Measured, same bits, interleaved
# isolated calls: Exaone layer 13.88 -> 13.56 us, fp32 tiny case 12.06 ->
# 11.84, batched GQA-8 60.91 -> 60.51, 64 new tokens 64.35 -> 63.13, MQA and
# the sq = 2 sweep at G = 8 unchanged.
KERNEL_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=3"]


def build(verbose: bool = False) -> str:
    objs = []
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        lang = (KERNEL_FLAGS + ["-x", "hip"]) if src.endswith(".hip") else []
        cmd = [HIPCC] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include")] + lang + \
            ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(ln for ln in (r.stderr or "").splitlines()
                         if "packed-fp32-ops" not in ln)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, errs))
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
