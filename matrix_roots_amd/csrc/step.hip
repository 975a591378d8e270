// The step around the preconditioner, both HBM-bound streams over float32
// matrices:
//
//  * momentum EMA, M <- mu M + (1 - mu) G, the momentum whose preconditioned
//    direction the optimizer applies (EMA-Gram page, section "Results");
//  * the MuonH hyperball update (ai.thesatyajit.com, "Marin 535B-A23B",
//    section "A sphere for every matrix"): c = lr ||W|| / max(||U||, 1e-10),
//    W' = W - c U,
//    W <- W' ||W|| / max(||W'||, 1e-10), norms over the whole matrix.
//
// The hyperball update makes two passes instead of three: the first reduces
// ||W||^2, ||U||^2 and <W, U> per block of rows (float64 partials), the
// second gets ||W'||^2 = ||W||^2 - 2 c <W, U> + c^2 ||U||^2 from them and
// writes (W - c U) ||W|| / ||W'|| in place; every block of a matrix sums that
// matrix's partials in the same fixed order, so the result is deterministic.
#include <math.h>

#include "launch.hpp"
#include "mr_common.hpp"
#include "step.hpp"

namespace mr {

namespace {

__device__ __forceinline__ int find_stream_job(const StreamBatch& B, int64_t b) {
  int jx = 0;
  while (jx + 1 < B.njobs && b >= B.job[jx + 1].block_begin) ++jx;
  return jx;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// Visit elements (r, c) of rows [r0, r1) of an m x n pair of matrices, VEC
// consecutive columns per call (VEC = 4: n, both leading dimensions and both
// pointers 16-byte compatible).
template <int VEC, typename F>
__device__ __forceinline__ void for_rows(int r0, int r1, int n, F&& f) {
  const int per_row = n / VEC;
  const int64_t total = (int64_t)(r1 - r0) * per_row;
  for (int64_t i = threadIdx.x; i < total; i += 256) {
    const int r = r0 + (int)(i / per_row);
    const int c = (int)(i % per_row) * VEC;
    f(r, c);
  }
}

}  // namespace

template <int VEC>
__global__ __launch_bounds__(256) void momentum_kernel(const StreamBatch B, double mu) {
  const int64_t b = blockIdx.x;
  const StreamJob& J = B.job[find_stream_job(B, b)];
  const int r0 = (int)(b - J.block_begin) * J.rows_per_block;
  const int r1 = min(J.m, r0 + J.rows_per_block);
  const float* G = J.in;
  float* M = J.inout;
  const double nu = 1.0 - mu;
  for_rows<VEC>(r0, r1, J.n, [&](int r, int c) {
    if constexpr (VEC == 4) {
      const float4 g = *reinterpret_cast<const float4*>(G + (int64_t)r * J.ld_in + c);
      float4* mp = reinterpret_cast<float4*>(M + (int64_t)r * J.ld_inout + c);
      float4 m = *mp;
      m.x = (float)(mu * (double)m.x + nu * (double)g.x);
      m.y = (float)(mu * (double)m.y + nu * (double)g.y);
      m.z = (float)(mu * (double)m.z + nu * (double)g.z);
      m.w = (float)(mu * (double)m.w + nu * (double)g.w);
      *mp = m;
    } else {
      float* mp = M + (int64_t)r * J.ld_inout + c;
      *mp = (float)(mu * (double)*mp + nu * (double)G[(int64_t)r * J.ld_in + c]);
    }
  });
}

// Pass 1: per block of rows, sum of W^2, U^2 and W U (float64).
template <int VEC>
__global__ __launch_bounds__(256) void hyperball_reduce_kernel(const StreamBatch B) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const StreamJob& J = B.job[find_stream_job(B, b)];
  const int blk = (int)(b - J.block_begin);
  const int r0 = blk * J.rows_per_block;
  const int r1 = min(J.m, r0 + J.rows_per_block);
  const float* W = J.inout;
  const float* U = J.in;
  double ww = 0.0, uu = 0.0, wu = 0.0;
  for_rows<VEC>(r0, r1, J.n, [&](int r, int c) {
    if constexpr (VEC == 4) {
      const float4 w = *reinterpret_cast<const float4*>(W + (int64_t)r * J.ld_inout + c);
      const float4 u = *reinterpret_cast<const float4*>(U + (int64_t)r * J.ld_in + c);
      ww += (double)w.x * w.x + (double)w.y * w.y + (double)w.z * w.z + (double)w.w * w.w;
      uu += (double)u.x * u.x + (double)u.y * u.y + (double)u.z * u.z + (double)u.w * u.w;
      wu += (double)w.x * u.x + (double)w.y * u.y + (double)w.z * u.z + (double)w.w * u.w;
    } else {
      const double w = W[(int64_t)r * J.ld_inout + c], u = U[(int64_t)r * J.ld_in + c];
      ww += w * w;
      uu += u * u;
      wu += w * u;
    }
  });
  ww = block_sum(ww, red);
  uu = block_sum(uu, red);
  wu = block_sum(wu, red);
  if (threadIdx.x == 0) {
    double* p = B.partial + (int64_t)J.slot * B.partial_stride + 3 * blk;
    p[0] = ww;
    p[1] = uu;
    p[2] = wu;
  }
}

// Pass 2: the matrix's norms from its partials, then W <- (W - c U) s.
template <int VEC>
__global__ __launch_bounds__(256) void hyperball_update_kernel(const StreamBatch B, double lr, double* norms) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const StreamJob& J = B.job[find_stream_job(B, b)];
  const int blk = (int)(b - J.block_begin);
  const double* p = B.partial + (int64_t)J.slot * B.partial_stride;
  double ww = 0.0, uu = 0.0, wu = 0.0;
  for (int i = threadIdx.x; i < J.nblocks; i += 256) {
    ww += p[3 * i];
    uu += p[3 * i + 1];
    wu += p[3 * i + 2];
  }
  ww = block_sum(ww, red);
  uu = block_sum(uu, red);
  wu = block_sum(wu, red);
  const double wn = sqrt(ww), un = sqrt(uu);
  const double c = lr * wn / fmax(un, 1e-10);
  const double pn = sqrt(fmax(ww - 2.0 * c * wu + c * c * uu, 0.0));
  const double s = wn / fmax(pn, 1e-10);
  if (blk == 0 && threadIdx.x == 0 && norms) {
    norms[3 * J.problem + 0] = wn;
    norms[3 * J.problem + 1] = un;
    norms[3 * J.problem + 2] = pn;
  }
  const int r0 = blk * J.rows_per_block;
  const int r1 = min(J.m, r0 + J.rows_per_block);
  float* W = J.inout;
  const float* U = J.in;
  for_rows<VEC>(r0, r1, J.n, [&](int r, int cc) {
    if constexpr (VEC == 4) {
      float4* wp = reinterpret_cast<float4*>(W + (int64_t)r * J.ld_inout + cc);
      const float4 u = *reinterpret_cast<const float4*>(U + (int64_t)r * J.ld_in + cc);
      float4 w = *wp;
      w.x = (float)(((double)w.x - c * u.x) * s);
      w.y = (float)(((double)w.y - c * u.y) * s);
      w.z = (float)(((double)w.z - c * u.z) * s);
      w.w = (float)(((double)w.w - c * u.w) * s);
      *wp = w;
    } else {
      float* wp = W + (int64_t)r * J.ld_inout + cc;
      *wp = (float)(((double)*wp - c * (double)U[(int64_t)r * J.ld_in + cc]) * s);
    }
  });
}

// ------------------------------------------------------------ launchers
hipError_t launch_momentum(const StreamBatch& b, int vec, double mu, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (vec == 4)
    hipLaunchKernelGGL(momentum_kernel<4>, dim3(b.total_blocks), dim3(256), 0, s, b, mu);
  else
    hipLaunchKernelGGL(momentum_kernel<1>, dim3(b.total_blocks), dim3(256), 0, s, b, mu);
  return hipGetLastError();
}

hipError_t launch_hyperball_reduce(const StreamBatch& b, int vec, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (vec == 4)
    hipLaunchKernelGGL(hyperball_reduce_kernel<4>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(hyperball_reduce_kernel<1>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_hyperball_update(const StreamBatch& b, int vec, double lr, double* norms, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (vec == 4)
    hipLaunchKernelGGL(hyperball_update_kernel<4>, dim3(b.total_blocks), dim3(256), 0, s, b, lr, norms);
  else
    hipLaunchKernelGGL(hyperball_update_kernel<1>, dim3(b.total_blocks), dim3(256), 0, s, b, lr, norms);
  return hipGetLastError();
}

}  // namespace mr
