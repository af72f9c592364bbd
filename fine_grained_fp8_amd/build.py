"""Build libfp8bs.so in-tree with hipcc for gfx950.

    python -m fine_grained_fp8_amd.build

Every call recompiles.  Flags that matter for the numerics: FP contraction
off (every rounding is the one written), FP32 denormals kept, correctly
rounded FP32 division, and no packed-FP32 instructions.  For speed: MFMA
results are kept in VGPRs.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp8bs.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "payload.hip", "accum.hip", "tiles.hip", "probe.hip", "fused.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results (the per-K-block partial sums) in VGPRs, where the FP32
    # scale fold reads them, instead of AGPRs plus a copy per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8bs.so)")


def build(verbose: bool = False) -> str:
    """Compile the library; returns its path.  Raises on compiler failure."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
