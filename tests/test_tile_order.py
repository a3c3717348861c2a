"""The digit GEMM's lower-triangle tile order (csrc/tile_order.h), compiled
for the host: for every tile-row count up to 130 it enumerates each tile with
tc <= tr exactly once, and the count is tm (tm + 1) / 2."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_quantization_solver_amd", "csrc")

DRIVER = r'''
#include <cstdio>
#include <vector>
#include "tile_order.h"
int main() {
  for (int tm = 1; tm <= 130; ++tm) {
    const int T = mpq::dg_lower_tiles(tm);
    if (T != tm * (tm + 1) / 2) {
      std::printf("count: tm %d gives %d\n", tm, T);
      return 1;
    }
    std::vector<char> seen((size_t)tm * tm, 0);
    for (int t = 0; t < T; ++t) {
      int tr = -1, tc = -1;
      mpq::dg_lower_tile(t, tm, tr, tc);
      if (tr < 0 || tr >= tm || tc < 0 || tc > tr || seen[(size_t)tr * tm + tc]++) {
        std::printf("tile: tm %d, t %d -> (%d, %d)\n", tm, t, tr, tc);
        return 1;
      }
    }
  }
  std::printf("ok\n");
  return 0;
}
'''


def test_lower_tile_order_enumerates_each_lower_tile_once(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "order.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "order"
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout
