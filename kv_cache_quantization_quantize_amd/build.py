"""Build libkivi.so (the HIP library) in-tree for gfx950.

    python -m kv_cache_quantization_quantize_amd.build

Always recompiles.  Flags that decide what the kernels compute:
  -ffp-contract=off   q*scale + zero stays two roundings (no FMA)
  no fast-math        IEEE division, round-to-nearest-even, denormals kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from emitting packed fp32 VALU ops
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkivi.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the attend's accumulators live across a loop
    # with a conditional rescale, and AGPR accumulators cost copies every step
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compiles every source to an object in parallel (one compiler process
    per file), then links the shared library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="kivi_build_") as obj_dir:
        objs = [os.path.join(obj_dir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[hipcc, *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
                for src, obj in zip(srcs, objs)]
        if verbose:
            for cmd in cmds:
                print(" ".join(cmd), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            codes = list(pool.map(lambda c: subprocess.run(c).returncode, cmds))
        failed = [src for src, rc in zip(srcs, codes) if rc != 0]
        if failed:
            raise subprocess.CalledProcessError(1, "hipcc -c " + " ".join(failed))
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
