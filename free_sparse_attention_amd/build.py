"""Build libfsa.so (gfx950) in-tree with hipcc.

    python -m free_sparse_attention_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep fp32 arithmetic on scalar (non-packed) vector instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfsa.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
