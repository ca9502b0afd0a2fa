"""Compile the HIP library (libreplayssm.so) in-tree for gfx950.

    python -m linear_attention_decode_replay_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libreplayssm.so")
SOURCES = ["rs_kernels.hip", "rs_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # No packed-fp32 instructions (v_pk_fma/mul/add_f32) in the gfx950 code:
    # turn the target feature off for the device pass.  hipcc hands the same
    # flag to the host (x86) pass, which warns that it does not know the
    # feature and ignores it; the device pass honours it
    # (tests/test_build_flags.py disassembles the built library to check).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core (MFMA) operands and results in ordinary VGPRs, not AGPRs:
    # the one MFMA in the library (the fp16-state flush fold) then accumulates
    # in the registers that already hold the tile, instead of copying it to
    # accumulation registers that count against the same budget (measured:
    # the Gated DeltaNet 128 x 128 fp16 kernel at 126 VGPRs + 64 AGPRs, two
    # waves per SIMD, against 126 VGPRs and four).
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
