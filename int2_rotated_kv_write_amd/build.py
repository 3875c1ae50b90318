"""Build the gfx950 shared library in-tree with hipcc.

    python -m int2_rotated_kv_write_amd.build

Produces int2_rotated_kv_write_amd/liboscar_gfx950.so from csrc/*.hip and
csrc/*.cpp.  Packed FP32 instructions are switched off for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liboscar_gfx950.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["oscar_api.hip", "kv_write.hip", "decode.hip", "decode_bf16.hip", "decode_noalloc.hip", "calibrate.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode loop rescales them with
    # VALU ops, which AGPR accumulators would turn into copies every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # device code only: no NaN operands, so max/min need no canonicalising moves
    # (the softmax max reductions become single DPP max instructions); host
    # code keeps its NaN checks on user arguments
    "-Xarch_device", "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
    # inline assembly must not clobber reserved registers (M0 is saved and restored
    # inside the statements that write it)
    "-Werror=inline-asm",
]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source into one shared library; always rebuilds."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
