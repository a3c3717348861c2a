"""Compile the HIP sources of the MPQ solver into an in-tree shared library.

    python -m post_quantization_solver_amd.build

produces post_quantization_solver_amd/libmpq.so for gfx950 (MI355X).  hipcc
cross-compiles, so no GPU is needed to build.  Each source is compiled to its
own object (in parallel; no device code crosses translation units), then the
objects are linked.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmpq.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "gemm64.hip", "rowops.hip", "scalar.hip", "lattice.hip", "cd.hip", "cd_lattice.hip",
           "chol.hip", "greedy.hip", "frontend.hip", "e8dp.hip", "probe.hip", "digitgemm.hip"]
ARCH = os.environ.get("MPQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc(), *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = [(c, r) for c, r in zip(cmds, results) if r.returncode != 0]
    for c, r in failed:
        sys.stderr.write(" ".join(c) + "\n" + r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed compiling " + ", ".join(os.path.basename(c[-3]) for c, _ in failed))
    tmp = LIB + ".tmp"
    res = _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libmpq.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
