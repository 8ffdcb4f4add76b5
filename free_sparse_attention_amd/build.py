"""Build libfsa.so (gfx950) in-tree with hipcc, and its LDS-poison debug twin.

    python -m free_sparse_attention_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libfsa.so")
# Debug build: every kernel fills its LDS with a NaN pattern at the start and
# between stages that reuse it (-DFSA_DEBUG_POISON_LDS); tests only.
POISON_LIB = os.path.join(PKG, "libfsa_poison.so")
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
    """Compile every HIP source into libfsa.so and, in parallel, into
    libfsa_poison.so (always recompiles both).  Returns the release library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = []
    for out, extra in ((LIB, []), (POISON_LIB, ["-DFSA_DEBUG_POISON_LDS"])):
        tmp = out + f".tmp{os.getpid()}"
        cmd = [hipcc, *HIPCC_FLAGS, *extra, "-o", tmp, *sources()]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = []
    for out, tmp, p in jobs:
        so, se = p.communicate()
        if p.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({p.returncode}):\n{so}\n{se}")
            if os.path.exists(tmp):
                os.remove(tmp)
        else:
            os.replace(tmp, out)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
