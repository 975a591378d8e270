// Polar orthogonalisation with the CANS coefficients: shared host/device
// definitions.
//
// tilderesearch, "Online KL Shampoo", section 2.3: the CANS polynomials were
// built for Muon's polar factor.  Each step X <- a_k X + b_k X X^T X moves
// every singular value by s <- s (a_k + b_k s^2) and keeps the singular
// vectors, i.e. p = s^2 follows the same recurrence p <- p (a_k + b_k p)^2
// as P = Z Y in the coupled inverse square root (cans.hpp), so the same
// suprema bound the spectral norms: ||X_k|| <= sqrt(p_k), ||X_k^T X_k|| <=
// p_k.  From X0 = G / sqrt(L), L = 1.01 ||G||_F^2, ten steps give
// U phi(Sigma / sqrt(L)) V^T, the polar factor U V^T to 3e-5 for singular
// values with sigma^2 / L in [1e-6, 0.99].
//
// The iteration runs on the tall orientation T (M x N, M >= N: G itself, or
// G^T for a wide G), keeping T and T^T so that both products are NT:
//   A  = T^T T          (N x N, symmetric: upper tiles, contraction over M)
//   T' = a T + b T A    (M x N, every tile, stored with its transpose)
#pragma once

#include "cans.hpp"

namespace mr {

// Per-matrix region: four split arrays (fp16 hi, then lo): T for even and odd
// steps (M x N), T^T (N x M), A (N x N).
__host__ __device__ inline int64_t polar_matrix_bytes(int64_t M, int64_t N) { return 4 * (3 * M * N + N * N); }

struct PolarClass {
  char* region;  // first matrix of the class
  int64_t matrix_bytes;
  int32_t M, N, count, TM, TN, U;  // U = TN (TN + 1) / 2 upper tiles of A
  int32_t slot_begin, block_begin, blocks_per_matrix, nblocks;
};

struct PolarLaunch {
  PolarClass cls[kMaxClasses];
  const RootState* state;
  double alpha, beta;  // stage A: alpha; stage X: T' = beta T + alpha T A
  int32_t ncls, total_blocks, stage, k;
};
enum PolarStage { kPolarA = 0, kPolarX = 1 };

// One matrix of a polar call, as the per-matrix kernels see it.
struct PolarJob {
  const float* G;
  int64_t ldg;
  float* O;
  int64_t ldo;
  char* region;
  int32_t m, n;
  int32_t slot, problem;
  int32_t block_begin, nblocks;
};
static_assert(sizeof(PolarJob) * kMaxRootJobs + 64 < 4096, "polar table fits the kernel arguments");
struct PolarBatch {
  PolarJob job[kMaxRootJobs];
  RootState* state;
  double* partial;
  int64_t partial_stride;
  int32_t njobs, total_blocks;
};

hipError_t launch_polar_stats(const PolarBatch& b, hipStream_t s);
hipError_t launch_polar_bound(RootState* state, const double* partial, int64_t stride, int32_t nslots,
                              double out_scale, hipStream_t s);
hipError_t launch_polar_init(const PolarBatch& b, double s0, hipStream_t s);
hipError_t launch_polar_gemm(const PolarLaunch& L, int vec, int prec, hipStream_t s);
int polar_tile(int prec, int stage);  // output tile side of a GEMM stage (prec 1: fp16, 3: split)
hipError_t launch_polar_finalize(const PolarBatch& b, double inv_sa9, hipStream_t s);

}  // namespace mr
