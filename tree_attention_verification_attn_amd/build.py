"""Builds libtreeverify.so (HIP for gfx950) in the package directory with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtreeverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in arch VGPRs: the softmax and the output rescale operate on them
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source into one shared library (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if verbose:
        noise = "is not a recognized feature for this target"
        print("\n".join(l for l in res.stderr.splitlines() if noise not in l))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
