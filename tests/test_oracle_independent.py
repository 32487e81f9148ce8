"""The CPU oracle and the input generators run without the HIP library.

A fresh interpreter imports ``oracle`` and ``workloads``, quantizes a small
tensor with the oracle, and then checks its own memory map: neither
``libmx.so`` nor anything from the ``block_scaled_bit_amd`` package may be
loaded, so the oracle's pins never depend on the code they check.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
import numpy as np
import oracle
import workloads
x = workloads.weights_small(rows=4, cols=64)
codes, scales, _ = oracle.quantize(oracle.FP6_E2M3, x)
assert codes.shape == (4, 2, 24) and scales.shape == (4, 2)
assert "block_scaled_bit_amd" not in sys.modules
with open("/proc/self/maps") as f:
    maps = f.read()
assert "libmx.so" not in maps, "libmx.so is mapped"
assert "liboracle.so" in maps
print("independent")
"""


def test_oracle_and_generators_load_without_the_library():
    env = dict(os.environ, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("independent")
