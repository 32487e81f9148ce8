"""Build the test-only probe library (tests/hwprobe/libcvtprobe.so): the
conversion and matrix-core probes, the library's fixed exponentials applied
element by element, and the byte-mix copy the benchmark times as its
ceiling."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libcvtprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "block_scaled_bit_amd", "csrc"),
           "-o", LIB + ".tmp", os.path.join(HERE, "cvt_probe.hip"), os.path.join(HERE, "mfma_probe.hip"),
           os.path.join(HERE, "bw_probe.hip"), os.path.join(HERE, "exp_probe.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
