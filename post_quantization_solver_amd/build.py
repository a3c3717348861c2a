"""Compile the HIP sources of the MPQ solver into an in-tree shared library.

    python -m post_quantization_solver_amd.build

produces post_quantization_solver_amd/libmpq.so for gfx950 (MI355X).  hipcc
cross-compiles, so no GPU is needed to build.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmpq.so")
SOURCES = ["api.hip", "gemm.hip", "gemm64.hip", "rowops.hip", "scalar.hip", "lattice.hip", "cd.hip", "cd_lattice.hip",
           "chol.hip", "greedy.hip", "frontend.hip", "e8dp.hip", "probe.hip"]
ARCH = os.environ.get("MPQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA sources/results in ordinary VGPRs: no accumulator-register copies
    # between the matrix cores and the VALU work that consumes their results
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmpq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
