"""Build libbatq.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbatq.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    # bit-exact fp32 chains: no contraction into FMA beyond the explicit ones,
    # fp32 denormals kept
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = ("packed-fp32-ops", "not a recognized feature")
    for line in (res.stdout + res.stderr).splitlines():
        if verbose or not any(n in line for n in noise):
            if line.strip():
                print(line, file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-4:])}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object, then link the shared library; raises on any
    compiler error."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        _run([hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    # (every symbol resolved at link time: a kernel whose host stub is missing fails here)
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
