"""Build libmx.so (the C-ABI library of include/mx.h) for gfx950 with hipcc.

Run ``python -m block_scaled_bit_amd.build`` (or ``__graft_entry__.build()``).
The library is built in-tree next to this file so that it travels with the
source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["mx_api.cpp", "mx_kernels.hip", "mx_attention.hip"]

# Device flags: gfx950 only; no floating-point contraction (every fused
# multiply-add in the kernels is written out); no packed-fp32 instruction
# selection; denormals are kept (the default; never -fgpu-flush-denormals).
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str, source: str = "mx_kernels.hip") -> str:
    """Write the gfx950 assembly of one source (for inspection)."""
    cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] + [
        "-S", "--offload-device-only", "-o", out_path, os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
