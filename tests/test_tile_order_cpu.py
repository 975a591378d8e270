"""Host checks of the device tile enumerations in mr_common.hpp, compiled
with the library's own compiler and run on the CPU:
  * upper_pair (the init kernels' workgroup -> tile pair map) visits the
    upper triangle of a T x T tile grid row by row, each pair once;
  * upper_tile_grouped (the symmetric GEMM tiles' banded order) visits every
    upper tile exactly once."""

import os
import subprocess

from matrix_roots_amd import build as mb

CHECK = r"""
#include "mr_common.hpp"
#include <cstdio>
#include <vector>
int main() {
  int bad = 0;
  std::vector<int> Ts;
  for (int T = 1; T <= 300; ++T) Ts.push_back(T);
  for (int T : {511, 512, 1000, 1024, 1448, 2047, 2048}) Ts.push_back(T);
  for (int T : Ts) {
    const int n = T * (T + 1) / 2;
    int pi = 0, pj = -1;
    for (int u = 0; u < n; ++u) {
      int bi, bj;
      mr::upper_pair(u, T, bi, bj);
      int ei = pi, ej = pj + 1;
      if (ej >= T) { ei = pi + 1; ej = ei; }
      if (bi != ei || bj != ej) {
        if (bad < 5) std::printf("upper_pair T=%d u=%d: (%d,%d), expected (%d,%d)\n", T, u, bi, bj, ei, ej);
        ++bad;
      }
      pi = ei; pj = ej;
    }
    if (T <= 512) {
      std::vector<char> seen((size_t)T * T, 0);
      for (int u = 0; u < n; ++u) {
        int ti, tj;
        mr::upper_tile_grouped(u, T, ti, tj);
        if (ti < 0 || tj >= T || ti > tj || seen[(size_t)ti * T + tj]) {
          if (bad < 5) std::printf("upper_tile_grouped T=%d u=%d: (%d,%d)\n", T, u, ti, tj);
          ++bad;
          continue;
        }
        seen[(size_t)ti * T + tj] = 1;
      }
    }
  }
  std::printf("%s\n", bad ? "FAIL" : "OK");
  return bad != 0;
}
"""


def test_tile_enumerations(tmp_path):
    src = tmp_path / "check.hip"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    cmd = [mb.hipcc(), "-O2", "-std=c++17", f"--offload-arch={mb.ARCH}", "-I", mb.CSRC, "-x", "hip", str(src),
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), run.stdout[-2000:]
