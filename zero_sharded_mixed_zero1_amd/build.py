"""Build libzero1.so (gfx950) in-tree with hipcc.

Flags that the arithmetic contract depends on:
  -ffp-contract=off      no fused multiply-add is formed from a*b+c (host and device)
  -packed-fp32-ops off   no v_pk_{add,mul,fma}_f32 is generated
fp32 division and square root stay correctly rounded (the HIP default), and
nothing flushes subnormals.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzero1.so")
SOURCES = [os.path.join(HERE, "csrc", "api.cpp"), os.path.join(HERE, "csrc", "kernels.hip"),
           os.path.join(HERE, "csrc", "static_ws.hip")]
# bandwidth calibration kernels used by bench.py (not part of the step library)
CALIB_LIB = os.path.join(HERE, "libzero1_calib.so")
CALIB_SOURCES = [os.path.join(HERE, "csrc", "calib.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include")]


def _hipcc(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile libzero1.so and the calibration library (always recompiles)."""
    _hipcc(SOURCES, LIB, verbose)
    _hipcc(CALIB_SOURCES, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
