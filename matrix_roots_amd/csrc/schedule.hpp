// Iteration schedule of the coupled Newton inverse p-th root (host and device).
//
// Every eigenvalue m of the iterate M follows m <- m * ((p + 1 - m) / p)^p.
// On [0, 1] the map is increasing with fixed point 1 and zero derivative
// there, so starting from the smallest normalised eigenvalue m0 (a lower bound
// eps / c) the count of steps until 1 - m <= tol serves every eigenvalue.
// For p = 2 this is the scalar recurrence behind the coupled Newton-Schulz
// iteration of tilderesearch, "Online KL Shampoo", section 2.2.
#pragma once

#include <hip/hip_runtime.h>

namespace mr {

__host__ __device__ inline double newton_scalar_step(int p, double m) {
  const double t = ((double)(p + 1) - m) / (double)p;
  double tp = t;
  for (int i = 1; i < p; ++i) tp *= t;
  return m * tp;
}

// K: iterations until 1 - m_K <= tol (at most cap, at least 1).
// j: first iteration index whose input eigenvalue floor m_j >= switch_m
//    (iterations t < j run in float64); j <= K.
__host__ __device__ inline void newton_schedule(double m0, double tol, double switch_m, int cap, int* K,
                                                int* j) {
  double m = m0;
  int k = 0;
  int jj = (m >= switch_m) ? 0 : -1;
  while (1.0 - m > tol && k < cap) {
    m = newton_scalar_step(4, m);
    ++k;
    if (jj < 0 && m >= switch_m) jj = k;
  }
  if (k == 0) k = 1;
  *K = k;
  *j = (jj < 0 || jj > k) ? k : jj;
}

}  // namespace mr
