// Inverse square root S^(-1/2) by the scaled CANS coupled Newton-Schulz
// iteration: shared host/device definitions (coefficients, step scales,
// launch descriptors).
//
// tilderesearch, "Online KL Shampoo", sections 2.2-2.4 and appendix D:
// from Y0 = S/L (L >= lambda_max(S)), Z0 = I, ten steps of
//   P_k = Z_k Y_k,  Q_k = a_k I + b_k P_k,  Y_{k+1} = Y_k Q_k,  Z_{k+1} = Q_k Z_k
// with the Chebyshev-optimised (CANS) pairs (a_k, b_k) below, then
// S^(-1/2) = Z_10 / sqrt(L).  Every eigenvalue y0 of Y0 follows the scalar
// recurrence y <- y q, z <- z q, q = a + b z y, so the suprema of y_k, z_k and
// p_k = z_k y_k over y0 in (0, 1] bound the spectral norms (hence every
// entry) of the symmetric intermediates.  Each intermediate is stored times a
// power of two that brings that bound to at most 2^14, inside the fp16 range
// (the page's per-step range scaling, section 2.4, with exact power-of-two
// factors).
#pragma once

#include <math.h>
#include <stdint.h>

#include "launch.hpp"

namespace mr {

constexpr int kCansSteps = 10;
constexpr int32_t kCansMethod = 16;     // RootState::method of these matrices
constexpr double kCansResidualRms = 0.1;  // NOT_CONVERGED above this rms of P_9 - I

// The page's CANS coefficient pairs (a_k, b_k), k = 0..9 (appendix D).
constexpr double kCansCoeff[kCansSteps][2] = {
    {5.182503604966906, -5.178098480082684},   {2.586120737395915, -0.6479542005271643},
    {2.567364126726186, -0.6454968804392178},  {2.520560084348265, -0.6393528082067044},
    {2.410759275435182, -0.6248683598710716},  {2.1883348130094173, -0.5952022073798908},
    {1.8595760874873613, -0.5504490972723968}, {1.589020160467417, -0.5126569802066718},
    {1.5051653981684994, -0.5007377068751799}, {1.5, -0.5},
};

// Suprema over y0 in (0, 1] of y_k, z_k (k = 0..10) and p_k (k = 0..10;
// p_10 = z_10 y_10), from the scalar recurrence on a dense grid (2^17
// log-spaced points in [1e-14, 1] and 2^17 evenly spaced in (0, 1]).
struct CansCeilings {
  double y[kCansSteps + 1], z[kCansSteps + 1], p[kCansSteps + 1];
};

inline CansCeilings cans_ceilings_compute() {
  CansCeilings c;
  for (int k = 0; k <= kCansSteps; ++k) c.y[k] = c.z[k] = c.p[k] = 0.0;
  const int n = 1 << 17;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < n; ++i) {
      const double y0 = pass == 0 ? pow(10.0, -14.0 + 14.0 * (double)i / (double)(n - 1))
                                  : (double)(i + 1) / (double)n;
      double y = y0, z = 1.0;
      for (int k = 0; k <= kCansSteps; ++k) {
        const double p = z * y;
        c.y[k] = fmax(c.y[k], fabs(y));
        c.z[k] = fmax(c.z[k], fabs(z));
        c.p[k] = fmax(c.p[k], fabs(p));
        if (k == kCansSteps) break;
        const double q = kCansCoeff[k][0] + kCansCoeff[k][1] * p;
        y *= q;
        z *= q;
      }
    }
  }
  return c;
}

// Power-of-two scale bringing a bound c to at most 2^14.
inline double cans_pow2_scale(double c) { return ldexp(1.0, (int)floor(14.0 - log2(c * 1.001))); }

struct CansScales {
  double sy[kCansSteps + 1], sz[kCansSteps + 1], sp[kCansSteps + 1];
};

inline CansScales cans_scales_from(const CansCeilings& c) {
  CansScales s;
  for (int k = 0; k <= kCansSteps; ++k) {
    s.sy[k] = cans_pow2_scale(c.y[k]);
    s.sz[k] = cans_pow2_scale(c.z[k]);
    s.sp[k] = cans_pow2_scale(c.p[k]);
  }
  return s;
}

// Launch stages of one step k:
//   kCansY1 (k = 0): Y1 = a0 Y0 + b0 Y0 Y0           (symmetric, one job)
//   kCansP  (k >= 1): P_k = Z_k Y_k, every tile, stored as P and P^T
//   kCansYZ (1 <= k <= 8): Y' = a Y + b Y P (= Y Z Y), Z' = a Z + b Z P^T (= Z Y Z)
//   kCansZ  (k = 9): Z' only
// Y Z Y and Z Y Z are symmetric whenever Y and Z are, commuting or not, so
// these two are upper-tile products with mirrored stores; P is not (rounding
// breaks the commutation) and is computed in full.
enum CansStage { kCansY1 = 0, kCansP = 1, kCansYZ = 2, kCansZ = 3 };

// Per-matrix region: six split arrays of d*d (fp16 hi at +0, lo at +2 d^2
// bytes, 4 d^2 bytes each): Y for even / odd k, Z for even / odd k, P, P^T.
constexpr int kCansBuffers = 6;
__host__ __device__ inline int64_t cans_matrix_bytes(int64_t d) { return (int64_t)kCansBuffers * 4 * d * d; }

struct CansClass {
  char* region;  // first matrix of the class
  int64_t matrix_bytes;
  int32_t d, count, T, U;
  int32_t slot_begin, block_begin, blocks_per_matrix, nblocks;
};

struct CansLaunch {
  CansClass cls[kMaxClasses];
  const RootState* state;
  double alpha[2], beta[2];  // job 0: Y1, P or Y'; job 1: Z'
  int32_t ncls, total_blocks, stage, k;
};

hipError_t launch_cans_bound(RootState* state, const double* partial, int64_t stride, int32_t nslots,
                             int32_t normalize, double eps, double z_out_scale, hipStream_t s);
hipError_t launch_cans_init(const RootBatch& b, double sy0, double za, double zb, hipStream_t s);
hipError_t launch_cans_gemm(const CansLaunch& L, int vec, int prec, hipStream_t s);
int cans_tile(int prec);  // output tile side of the GEMM launches of a precision (1: fp16, 3: split)
hipError_t launch_cans_finalize(const RootBatch& b, double inv_sp9, hipStream_t s);
hipError_t launch_cans_info(RootState* state, const double* partial, int64_t stride, int32_t count,
                            mr_root_info* info, double rms_limit, hipStream_t s);

}  // namespace mr
