"""Build libkivi.so (the HIP library) in-tree for gfx950.

    python -m kv_cache_quantization_quantize_amd.build

Always recompiles.  Flags that decide what the kernels compute:
  -ffp-contract=off   q*scale + zero stays two roundings (no FMA)
  no fast-math        IEEE division, round-to-nearest-even, denormals kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from emitting packed fp32 VALU ops
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkivi.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the attend's accumulators live across a loop
    # with a conditional rescale, and AGPR accumulators cost copies every step
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC,
           "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
