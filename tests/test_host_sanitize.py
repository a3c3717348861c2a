"""The library's host code (argument validation, workspace layout, codebook
recognition and table building) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only, and driven through those
paths by a small C program with no GPU involved."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import mpq_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "post_quantization_solver_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_host_code_under_sanitizers(tmp_path):
    from post_quantization_solver_amd import build as B
    out = tmp_path / "obj"
    out.mkdir()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")] + SAN
    cmds = [[HIPCC, *flags, "-c", os.path.join(PKG, "csrc", s), "-o", str(out / (s + ".o"))] for s in B.SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
    for c, r in zip(cmds, res):
        assert r.returncode == 0, " ".join(c) + "\n" + r.stderr[-3000:]
    exe = tmp_path / "driver"
    drv = tmp_path / "driver.o"
    r = subprocess.run([CLANG, "-c", "-x", "c", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host", "validation_driver.c"),
                        "-o", str(drv)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    link = [HIPCC, "-O1", "-g", f"--offload-arch={B.ARCH}", *SAN, str(drv),
            *[str(out / (s + ".o")) for s in B.SOURCES], "-ldl", "-o", str(exe)]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    K = 4096
    cbf = tmp_path / "e8.bin"
    S.e8_codebook(K).astype(np.float32).tofile(cbf)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe), str(cbf), str(K)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
