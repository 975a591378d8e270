// Two-sided application of the quarter powers on the float32 matrix cores.
//
//   U = alpha * XL * G * XR
//
// (marin.community, "Sharding EMA-Gram eigensolves", section "Background":
// the inverse quarter powers shape the update direction; the two-sided form
// is Shampoo's, tilderesearch "Online KL Shampoo", section 1.)
// Both products run as C = A * B^T on row-contiguous operands:
//   W^T = XR * G^T   (n x m; A = XR rows, B = G rows, contraction n)
//   U   = XL * W     (m x n; A = XL rows, B = W^T rows, contraction m)
// using the symmetry of XR and XL.  This file holds the generic float32
// job-batched kernel; the host runtime issues the two launches.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace mr {

template <int VEC>
__global__ __launch_bounds__(256, 2) void f32_nt_kernel(const F32Batch batch) {
  __shared__ float smem[F32Tile::LDS_FLOATS];

  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const F32Job& J = batch.job[jx];
  const int tile = (int)xcd_remap(b - J.block_begin, round8(J.nblocks));
  if (tile >= J.nblocks) return;
  int ti, tj;
  full_tile_grouped(tile, (J.M + F32Tile::BM - 1) / F32Tile::BM, J.tiles_n, ti, tj);
  const int m0 = ti * F32Tile::BM;
  const int n0 = tj * F32Tile::BN;

  v16f acc[2][2];
  f32_nt_tile<VEC>(J.A, J.lda, J.B, J.ldb, J.M, J.N, J.K, m0, n0, smem, acc);

  const float alpha = J.alpha;
  float* C = J.C;
  const int64_t ldc = J.ldc;
  const int M = J.M, N = J.N;
  f32_for_each(acc, [&](int r, int c, float v) {
    const int gr = m0 + r, gc = n0 + c;
    if (gr < M && gc < N) C[(int64_t)gr * ldc + gc] = alpha * v;
  });
}

hipError_t launch_f32_nt(const F32Batch& b, int vec, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (vec == 4)
    hipLaunchKernelGGL(f32_nt_kernel<4>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(f32_nt_kernel<1>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace mr
