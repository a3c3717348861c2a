"""Register budgets of the compiled kernels (host-only: hipcc emits the gfx950
code object's metadata without a GPU).

No kernel may use scratch memory: no vector-register spills and no private
arrays (scalar registers spill into vector-register lanes, which costs
instructions but no memory traffic, so those are allowed).  A spill inside
the digit GEMM's K loop turns every step's accumulator traffic into scratch
loads and stores: at 5 digits that made each c5 linear product 2.4 times
slower while every parity test still passed, so only this check can see it.
The digit GEMM also has to fit two waves per SIMD (at most 256 VGPRs, 8
waves per workgroup): its LDS stages allow one workgroup per CU, and one wave
per SIMD leaves the matrix cores idle at every barrier.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "post_quantization_solver_amd")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def kernel_metadata(src, out):
    from post_quantization_solver_amd import build as B
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    cmd = [B.hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    meta = text[text.index("amdhsa.kernels:"):text.index(".end_amdgpu_metadata")]
    kernels = {}
    for blk in re.split(r"\n  - ", meta)[1:]:
        # the kernel's own keys sit at four spaces; its arguments' keys are indented further
        fields = dict(re.findall(r"^ {4}\.(\w+):\s+(\S+)", "    " + blk, re.M))
        if "name" not in fields or "vgpr_count" not in fields:
            continue   # amdhsa.version and the like
        kernels[fields["name"]] = {k: int(fields[k]) for k in ("vgpr_count", "vgpr_spill_count", "private_segment_fixed_size")}
    return kernels


@pytest.fixture(scope="module")
def metadata(tmp_path_factory):
    from post_quantization_solver_amd import build as B
    tmp = tmp_path_factory.mktemp("isa")
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda s: (s, kernel_metadata(s, str(tmp / (s + ".s")))), B.SOURCES))
    return dict(res)


def test_no_kernel_uses_scratch_memory(metadata):
    spills = [(src, name, k["vgpr_spill_count"], k["private_segment_fixed_size"])
              for src, ks in metadata.items() for name, k in ks.items()
              if k["vgpr_spill_count"] or k["private_segment_fixed_size"]]
    assert not spills, spills
    assert sum(len(ks) for ks in metadata.values()) > 50


def test_digit_gemm_fits_two_waves_per_simd(metadata):
    gemms = {n: k for n, k in metadata["digitgemm.hip"].items() if "digit_gemm_kernel" in n}
    assert len(gemms) == 10   # 5 epilogues x 2 digit counts
    for name, k in gemms.items():
        assert k["vgpr_count"] <= 256, (name, k)
