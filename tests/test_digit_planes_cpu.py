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
