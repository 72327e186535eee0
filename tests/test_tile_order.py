"""The grouped GEMM's tile order inside an expert, checked on the host.

`grouped_tile_order` (csrc/gemm.h) maps a workgroup's position among an
expert's tiles to the (M tile, N tile) it computes. It must be a bijection for
every expert shape, or some output tile would go unwritten (or be written
twice); and with a multiple of 4 N tiles every run of one tile height must be a
multiple of 4 long, the property that spreads tile heights evenly over an XCD's
four shader engines. The function is compiled from the header's own text with
the host compiler; no GPU is involved.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_H = os.path.join(ROOT, "sparse_moe_layer_correction_amd", "csrc", "gemm.h")

DRIVER = r"""
#include <algorithm>
#include <cstdio>
#include <vector>
using std::min;
#define __host__
#define __device__
#define __forceinline__ inline
%s
int main() {
  long bad = 0, cases = 0, badrun = 0;
  for (int ne = 1; ne <= 40; ++ne)
    for (int tail = 0; tail <= 1; ++tail) {
      const int nfull = ne - tail;
      for (int ntl = 1; ntl <= 25; ++ntl)
        for (int gm : {1, 2, 3, 4, 8, 1 << 20}) {
          std::vector<int> seen(ne * ntl, 0);
          for (int l = 0; l < ne * ntl; ++l) {
            int mt = -1, nt = -1;
            grouped_tile_order(l, ne, nfull, ntl, gm, mt, nt);
            if (mt < 0 || mt >= ne || nt < 0 || nt >= ntl) { ++bad; continue; }
            seen[mt * ntl + nt]++;
          }
          for (int v : seen) bad += v != 1;
          ++cases;
          if (ntl %% 4 == 0) {   // runs of one height (short last M tile or not)
            int run = 0, prev = -1;
            for (int l = 0; l < ne * ntl; ++l) {
              int mt, nt;
              grouped_tile_order(l, ne, nfull, ntl, gm, mt, nt);
              const int h = tail && mt == ne - 1;
              if (h != prev && prev >= 0) { badrun += run %% 4 != 0; run = 0; }
              prev = h;
              ++run;
            }
            badrun += run %% 4 != 0;
          }
        }
    }
  std::printf("%%ld %%ld %%ld\n", cases, bad, badrun);
  return 0;
}
"""


def _function_source():
    src = open(GEMM_H, encoding="utf-8").read()
    m = re.search(r"^__host__ __device__ __forceinline__ void grouped_tile_order\(.*?^}\n", src, flags=re.S | re.M)
    assert m, "grouped_tile_order not found in gemm.h"
    return m.group(0)


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_grouped_tile_order_is_a_bijection_with_runs_of_four(tmp_path):
    cpp = tmp_path / "order.cpp"
    exe = tmp_path / "order"
    cpp.write_text(DRIVER % _function_source())
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), str(cpp)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    cases, bad, badrun = map(int, out)
    assert cases == 40 * 2 * 25 * 6
    assert bad == 0, f"{bad} tiles unmapped, out of range or mapped twice"
    assert badrun == 0, f"{badrun} runs of one tile height not a multiple of 4"
