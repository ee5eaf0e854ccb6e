"""Build libmla_mxfp4.so (host C++ + gfx950 HIP kernels) in-tree with hipcc.

Usage: ``python -m mla_mxfp4_kv_amd.build`` (or ``build()`` from Python).
The library lands next to this file so it travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmla_mxfp4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["mla_api.cpp", "mla_plan.cpp", "mla_kernels.hip", "mla_dense_kernels.hip", "mla_plan_kernel.hip", "mla_noalloc.hip", "mla_mxfp4_24_kernels.hip"]

# gfx950 only; packed-fp32 VALU forms are kept out of the generated code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: avoids AGPR<->VGPR copies around VALU work
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla_mxfp4.so)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link the shared library; returns its path."""
    inc = os.path.join(ROOT, "include")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", inc, "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_PATH)
