"""Build the HIP library in-tree: ``python -m vlm_multimodal_rotary_amd.build``.

Compiles csrc/*.hip and csrc/*.cpp for gfx950 with hipcc into
vlm_multimodal_rotary_amd/libmrope.so.  Packed-FP32 instruction selection is
disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmrope.so")
ARCH = os.environ.get("MROPE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["mrope_kernels.hip", "mrope_pipe.hip", "mrope_flat.hip", "mrope_planes.hip",
           "mrope_positions.hip", "mrope_copy.hip", "mrope_api.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = DEVICE
        else:
            cmd[1:1] = ["-D__HIP_PLATFORM_AMD__"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
