// Iteration schedules of the coupled Newton inverse p-th root (host and device).
//
// Coupled iteration: T = ((p+1) I - M/s)/p, X <- s^(-1/p) X T, M <- T^p M / s.
// For any scale s the invariant X^p M0 = M holds (all iterates are
// polynomials in M0 and commute), so X -> M0^(-1/p) once M -> I.  Every
// eigenvalue m of M follows the scalar map m <- g(m/s) with
// g(x) = x ((p+1-x)/p)^p, which rises on [0, 1] to its fixed point g(1) = 1
// and falls beyond 1.
//
// * s = 1 is the classical iteration: the smallest eigenvalue eps/c fixes the
//   count of steps until 1 - m <= tol.  For p = 2 this is the scalar recurrence
//   behind coupled Newton-Schulz (tilderesearch, "Online KL Shampoo",
//   section 2.2, roughly 21 iterations from a floor of 1e-6).
// * Per-step scales shorten the slow start.  The OKLS page (section 2.3) tunes
//   per-step polynomial coefficients of the coupled iteration for a fixed
//   step budget (CANS); it prints them for p = 2 only.  Here, for p = 4, the
//   scale of each step is chosen from the interval [l, u] that holds the
//   spectrum of M: s balances g(l/s) = g(u/s) (the best new floor for this
//   polynomial family), with u/s capped (kScaleCap64 while the steps run in
//   float64, kScaleCap32 after the switch), and the interval becomes
//   [min(g(l/s), g(u/s)), 1].  This needs bounds only, never the matrix.
#pragma once

#include <hip/hip_runtime.h>

namespace mr {

constexpr int kMaxNewtonIters = 100;
constexpr double kScaleCap64 = 4.8;  // cap on u/s while steps run in float64 (top-eigenvalue
                                     // errors grow ~95x per step there: harmless in float64)
constexpr double kScaleCap32 = 3.0;  // ... and in float32 (errors in the top
                                     // eigenvalues grow ~|1 - 4x/(5-x)| per step)

// Finishing step.  Once the spectrum of M lies in [1 - delta, 1], the root is
// X M^(-1/4) = X q(E) with E = I - M and q the Taylor polynomial of
// (1 - x)^(-1/4) (coefficients 1, 1/4, 5/32, 15/128, 195/2048); the relative
// error of X is max |(1 - x)^(1/4) q(x) - 1| over [0, delta].  Degree 2 costs
// one product for q(M) and one for X q; degree 4 costs three, E^2 and
// R = c2 + c3 E + c4 E^2 from one M M, then E^2 R and X q.  The limits keep
// that error below 5e-7 (the plain step stops at 1 - l <= 1e-6, whose X error
// is about 2.5e-7); past them the scaled step continues.
constexpr double kFinishQuad = 0.0162;
constexpr double kFinishQuartic = 0.0898;

__host__ __device__ inline double newton_scalar_step(int p, double m) {
  const double t = ((double)(p + 1) - m) / (double)p;
  double tp = t;
  for (int i = 1; i < p; ++i) tp *= t;
  return m * tp;
}

__host__ __device__ inline double g4(double x) {
  const double t = (5.0 - x) * 0.25;
  const double t2 = t * t;
  return x * t2 * t2;
}

// Scaled schedule for p = 4 from the spectrum bound [l, u] of M0, 0 < l <= u.
// Writes the step scales to s_out[0..K) (s_out may be null), returns K >= 1
// (steps until 1 - l <= tol, at most cap), j <= K, the first step whose
// input floor l >= switch_m (steps t < j run in float64), and fin, the
// degree in M of the last step's X update: 1 (the plain step, X only), or,
// with finish set, 2 or 4 (the Taylor finish above, taken at the first step
// t >= max(j, 1) whose floor allows it and whose plain step would not already
// end the iteration).
__host__ __device__ inline void newton_scaled_schedule(double l, double u, double tol, double switch_m, int cap,
                                                       double* s_out, int* K, int* j, bool finish = false,
                                                       int* fin = nullptr) {
  int k = 0;
  int jj = -1;
  int deg = 1;
  while (true) {
    if (jj < 0 && l >= switch_m) jj = k;
    if ((k > 0 && 1.0 - l <= tol) || k >= cap) break;
    // y = u/s in [1, min(cap, u/l)] with g(y) = g(y l/u), by bisection
    const double r = l / u;
    double hi = fmin(jj < 0 ? kScaleCap64 : kScaleCap32, 1.0 / r);
    double y;
    if (hi <= 1.0 || g4(hi) >= g4(hi * r)) {
      y = fmax(hi, 1.0);
    } else {
      double lo = 1.0;
      for (int it = 0; it < 80; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (g4(mid) - g4(mid * r) > 0.0)
          lo = mid;
        else
          hi = mid;
      }
      y = lo;
    }
    const double s = u / y;
    if (s_out) s_out[k] = s;
    const double a = g4(l / s), b = g4(u / s);
    const bool peak_inside = l / s <= 1.0 && u / s >= 1.0;
    const double l_next = fmin(a, b);
    if (finish && jj >= 0 && k > 0 && 1.0 - l_next > tol) {
      if (1.0 - l <= kFinishQuad) deg = 2;
      else if (1.0 - l <= kFinishQuartic) deg = 4;
      if (deg > 1) {
        ++k;
        break;
      }
    }
    l = l_next;
    u = peak_inside ? 1.0 : fmax(a, b);
    ++k;
  }
  if (k == 0) k = 1;
  *K = k;
  *j = (jj < 0 || jj > k) ? k : jj;
  if (fin) *fin = deg;
}

}  // namespace mr
