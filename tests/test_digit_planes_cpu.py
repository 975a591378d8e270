"""Host checks of the int8 digit planes the float64 Newton steps multiply
(gemm_i8.hpp), compiled with the library's own compiler and run on the CPU:
  * oz_digits writes six digits of at most 65 in magnitude whose weighted sum
    2^e sum_p d_p 2^-(6 + 7 p) is v rounded to the nearest multiple of
    2^(e - 41) (ties to even), for values over the whole exponent range, at
    the bound |v| = 2^e and at zero;
  * the product of two such matrices summed per anti-diagonal r = p + q <= 5
    with the weights 2^(eA + eB - 12 - 7 r), as the kernel combines its int32
    accumulators, matches the float64 product of the rounded matrices to the
    dropped pairs' size, and every partial sum stays inside int32 for
    K = 8192.
The expected values are computed here from the definition (exact integer
arithmetic in Python), not by the library."""

import math
import os
import subprocess
from fractions import Fraction

import numpy as np

from matrix_roots_amd import build as mb

CHECK = r"""
#include "gemm_i8.hpp"
#include <cstdio>
int main() {
  double v; int e;
  while (std::scanf("%lf %d", &v, &e) == 2) {
    int8_t dg[mr::kOzSlices];
    mr::oz_digits(v, e, dg);
    for (int p = 0; p < mr::kOzSlices; ++p) std::printf("%d ", (int)dg[p]);
    std::printf("\n");
  }
  return 0;
}
"""


def _digits(tmp_path, pairs):
    src = tmp_path / "digits.hip"
    src.write_text(CHECK)
    exe = tmp_path / "digits"
    cmd = [mb.hipcc(), "-O2", "-std=c++17", f"--offload-arch={mb.ARCH}", "-I", mb.CSRC, "-x", "hip", str(src),
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    inp = "".join(f"{v.hex()} {e}\n" for v, e in pairs)
    # %lf reads C99 hexadecimal floats: the values cross exactly
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    return [[int(x) for x in line.split()] for line in out if line.strip()]


def _expected(v, e):
    """v rounded to the nearest multiple of 2^(e - 41), ties to even, exactly."""
    x = Fraction(v) * Fraction(2) ** (41 - e)
    n = math.floor(x)
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return Fraction(n) * Fraction(2) ** (e - 41)


def test_digits_round_to_41_bits(tmp_path):
    rng = np.random.default_rng(7)
    pairs = []
    for _ in range(3000):
        e = int(rng.integers(-40, 4))
        pairs.append((float(rng.uniform(-1.0, 1.0)) * 2.0 ** e, e))
    for e in (-20, 0, 1, 2):
        pairs += [(2.0 ** e, e), (-(2.0 ** e), e), (0.0, e), (2.0 ** (e - 41) * 1.5, e), (2.0 ** (e - 41) * 2.5, e),
                  (2.0 ** (e - 42), e), (-(2.0 ** (e - 41)) * 0.5, e), (float(np.nextafter(2.0 ** e, 0.0)), e)]
    got = _digits(tmp_path, pairs)
    assert len(got) == len(pairs)
    for (v, e), dg in zip(pairs, got):
        assert len(dg) == 6 and max(abs(x) for x in dg) <= 65, (v, e, dg)
        rec = sum(Fraction(d) * Fraction(2) ** (e - 6 - 7 * p) for p, d in enumerate(dg))
        assert rec == _expected(v, e), (v, e, dg)


def test_anti_diagonal_product(tmp_path):
    rng = np.random.default_rng(11)
    n, K = 6, 40
    eA = rng.integers(-3, 2, n)
    eB = rng.integers(-3, 2, n)
    A = rng.uniform(-1, 1, (n, K)) * np.exp2(eA)[:, None]
    Bm = rng.uniform(-1, 1, (n, K)) * np.exp2(eB)[:, None]
    pairs = [(float(A[i, k]), int(eA[i])) for i in range(n) for k in range(K)]
    pairs += [(float(Bm[j, k]), int(eB[j])) for j in range(n) for k in range(K)]
    got = np.array(_digits(tmp_path, pairs), dtype=np.int64)
    DA = got[: n * K].reshape(n, K, 6)
    DB = got[n * K:].reshape(n, K, 6)
    Ar = np.array([[float(_expected(A[i, k], eA[i])) for k in range(K)] for i in range(n)])
    Br = np.array([[float(_expected(Bm[j, k], eB[j])) for k in range(K)] for j in range(n)])
    for i in range(n):
        for j in range(n):
            acc = [sum(int(DA[i, k, p]) * int(DB[j, k, r - p]) for k in range(K) for p in range(r + 1))
                   for r in range(6)]
            c = sum(Fraction(acc[r]) * Fraction(2) ** (int(eA[i] + eB[j]) - 12 - 7 * r) for r in range(6))
            exact = sum(Fraction(Ar[i, k]) * Fraction(Br[j, k]) for k in range(K))
            # dropped pairs p + q >= 6: |d| <= 65, weight 2^(eA + eB - 12 - 7 r), K terms each
            bound = Fraction(K * 65 * 65 * 7) * Fraction(2) ** (int(eA[i] + eB[j]) - 12 - 42)
            assert abs(c - exact) <= bound, (i, j, float(c - exact), float(bound))
    # int32 headroom of one anti-diagonal at K = 8192: at most 6 pairs of 65 x 65
    assert 6 * 8192 * 65 * 65 < 2 ** 31


LAYOUT = r"""
#include "root.hip"
#include <cstdio>
#include <vector>
struct Iv { long a, b; const char* what; };
static bool overlap(const Iv& x, const Iv& y) { return x.a < y.b && y.a < x.b; }
int main() {
  int bad = 0;
  std::vector<int> ds;
  for (int d = 33; d <= 600; ++d) ds.push_back(d);
  for (int d : {1024, 1056, 1184, 1248, 1536, 2048, 3072, 4096, 8192}) ds.push_back(d);
  for (int d : ds) {
    const mr::OzLayout ly = mr::oz_layout(d);
    const long d2 = (long)d * d, dp = mr::oz_pad(d);
    const long bytes = mr::oz_f64_bytes(d) + ly.extra;
    if (bytes % 256 != 0) { std::printf("d=%d: region %ld not a multiple of 256\n", d, bytes); ++bad; }
    for (int t = 0; t < 2; ++t) {
      char* R = nullptr;
      const mr::OzRegion z = mr::oz_region(R + 4096, d, t);  // offsets from a 4096-aligned base
      const mr::Roles64 r64 = mr::roles64(R + 4096, d, t);
      const mr::RolesS rs = mr::roless(R + 4096, d, t);
      auto off = [&](const void* p) { return (long)((const char*)p - (R + 4096)); };
      // live through a float64 step: M (float64), X, X', the split copy of M
      std::vector<Iv> live = {{off(r64.M), off(r64.M) + 8 * d2, "M f64"},
                              {off(rs.X.hi), off(rs.X.hi) + 4 * d2, "X"},
                              {off(rs.Xn.hi), off(rs.Xn.hi) + 4 * d2, "X'"},
                              {off(rs.Mx.hi), off(rs.Mx.hi) + 4 * d2, "Mx"}};
      std::vector<Iv> mine;
      for (int p = 0; p < mr::kOzSlices; ++p) {
        mine.push_back({off(z.M.p[p]), off(z.M.p[p]) + ly.plane, "M plane"});
        mine.push_back({off(z.T4.p[p]), off(z.T4.p[p]) + ly.plane, "T4 plane"});
        mine.push_back({off(z.T2.p[p]), off(z.T2.p[p]) + ly.plane, "T2 plane"});
      }
      mine.push_back({off(z.eM), off(z.eM) + 4 * dp, "exponents"});
      const Iv slot_next = {off(r64.T2), off(r64.T2) + 8 * d2, "M' slot"};
      for (size_t i = 0; i < mine.size(); ++i) {
        const Iv& x = mine[i];
        if (x.a < 0 || x.b > bytes || (x.a % 16) != 0) {
          std::printf("d=%d t=%d: %s [%ld,%ld) outside [0,%ld) or misaligned\n", d, t, x.what, x.a, x.b, bytes);
          ++bad;
        }
        for (const Iv& y : live)
          if (overlap(x, y)) { std::printf("d=%d t=%d: %s overlaps %s\n", d, t, x.what, y.what); ++bad; }
        // only T2's planes may sit in the slot M' is written to (after stage 1)
        if (x.what[0] != 'T' || x.what[1] != '2')
          if (overlap(x, slot_next)) { std::printf("d=%d t=%d: %s overlaps the M' slot\n", d, t, x.what); ++bad; }
        for (size_t j = i + 1; j < mine.size(); ++j)
          if (overlap(x, mine[j])) { std::printf("d=%d t=%d: %s overlaps %s\n", d, t, x.what, mine[j].what); ++bad; }
      }
    }
    if (bad > 20) break;
  }
  // the planes sit in the float64 slots where they fit (no growth for d % 128 == 0)
  if (mr::oz_layout(4096).extra != 16384 || mr::oz_layout(1024).extra != 4096) { std::printf("extra grew\n"); ++bad; }
  std::printf("%s\n", bad ? "FAIL" : "OK");
  return bad != 0;
}
"""


def test_plane_layout(tmp_path):
    """The digit planes of M, T2 and T4 and M's exponents never overlap each
    other or what a float64 step keeps live (M, X, X', the split copy of M),
    stay inside the region, are 16-byte aligned, and only T2's share the slot
    M' is written to; for d a multiple of 128 they add nothing but the
    exponents to the region."""
    src = tmp_path / "layout.hip"
    src.write_text(LAYOUT)
    exe = tmp_path / "layout"
    cmd = [mb.hipcc(), "-O1", "-std=c++17", f"--offload-arch={mb.ARCH}", "-I", mb.CSRC, "-x", "hip", str(src),
           "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("OK"), run.stdout[-3000:]
