"""Build libqgemm.so in-tree with hipcc for gfx950.

    python bit_weight_only_dequant_amd/build.py
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqgemm.so")
ARCH = os.environ.get("QGEMM_ARCH", "gfx950")

# No packed-fp32 instructions: they are kept out of every code object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    host_o = os.path.join(out_dir, "host.o")
    # host-only translation unit (no device code, no device flags)
    _run([hipcc, *COMMON, "-c", os.path.join(CSRC, "host.cpp"), "-o", host_o], verbose)
    objs = [host_o]
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        obj = os.path.join(out_dir, src[:-4] + ".o")
        _run([hipcc, *COMMON, f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
