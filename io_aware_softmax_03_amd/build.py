"""Compile the HIP sources into the in-tree shared library ``libfa.so`` (gfx950 only).

Usage: ``python -m io_aware_softmax_03_amd.build`` (or ``build()`` from Python).
Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked with hipcc.
Packed fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no NaNs are produced on the hot paths (masked scores are -inf, never NaN): drop the
    # NaN-quieting canonicalisations around v_max/v_max3 and run kernels with IEEE mode off
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


# Per-file extra flags. The forward kernel runs one wave per SIMD with 512 registers; by
# default the compiler then gives every MFMA the AGPR accumulator form, which would put the
# score tiles in AGPRs and cost a copy to VGPRs for each softmax step. With the VGPR form the
# output accumulators and scores sit in VGPRs and the Q operands in AGPRs.
# The FP8 forward kernel needs the same form to stay out of scratch memory. In the backward
# kernels the AGPR form copied every score, dP and dQ tile between the register files each
# step; there the dK, dV accumulators (the dK/dV kernel runs one wave per SIMD) are put in
# AGPRs by their own inline-assembly MFMAs instead.
FILE_FLAGS = {
    "fwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fwd_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
