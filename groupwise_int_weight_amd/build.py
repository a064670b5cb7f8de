"""Build libngq.so in-tree with hipcc for gfx950.

    python -m groupwise_int_weight_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libngq.so")

SOURCES = [os.path.join(CSRC, n) for n in ("ngq_host.cpp", "ngq_gemm.hip", "ngq_rescale.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the T > 8 kernels scale every MFMA
    # result on the VALU, which otherwise first copies it out of an AGPR
    # (one v_accvgpr_read per value); the decode kernels compile to the same
    # code either way
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
