"""Build step of libddtree.so: hipcc for gfx950, in-tree."""

from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "api.hip")
LIB = os.path.join(HERE, "libddtree.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # A wave's atomic add of per-lane amounts to one address: one DPP scan and
    # one atomic instead of a scalar loop over the active lanes.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*")) +
                  [os.path.join(ROOT, "include", "ddtree.h")])


def build_library(verbose: bool = False) -> str:
    """Compile csrc/api.hip (which includes the kernel headers) into libddtree.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB
