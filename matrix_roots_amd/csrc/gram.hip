// Gram EMA on the float64 matrix cores (SYRK with a fused EMA epilogue).
//
//   left:  S <- beta * S + (1 - beta) * G * G^T     (S is m x m)
//   right: S <- beta * S + (1 - beta) * G^T * G     (S is n x n)
//
// The exponential moving averages of gradient products that EMA-Gram keeps
// per linear weight (marin.community, "Sharding EMA-Gram eigensolves",
// section "Background").  float32 entries of G are widened to float64 on the
// way into LDS; their products are exact in float64 and are summed in float64
// by v_mfma_f64_16x16x4_f64.  Only the upper triangle of 128 x 128 tiles is
// computed; in full storage every computed element is written to both (i, j)
// and (j, i), so the state stays exactly symmetric and only its upper
// triangle is read; in packed storage (upper triangle by rows) each element
// is read and written once.
#include "gemm_core.hpp"
#include "launch.hpp"

// Direct-to-LDS float32 operands (f64g_tile) where K is a multiple of 16 and
// rows are 16-byte aligned; kSyrkStages stages.
constexpr int kSyrkStages = 3;

namespace mr {

template <bool RIGHT, typename TS, int VEC>
__global__ __launch_bounds__(256, 2) void syrk_ema_kernel(const SyrkBatch batch) {
  __shared__ __attribute__((aligned(16))) double smem[F64Tile::LDS_DOUBLES];

  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const SyrkJob& J = batch.job[jx];
  const int ntiles = J.T * (J.T + 1) / 2;
  const int local = (int)xcd_remap(b - J.block_begin, round8(ntiles));
  if (local >= ntiles) return;
  int ti, tj;
  upper_tile_grouped(local, J.T, ti, tj);
  const int m0 = ti * F64Tile::BM, n0 = tj * F64Tile::BN;

  v4d acc[4][4];
  if (VEC == 4 && J.K % 16 == 0) {
    static_assert(F64G<RIGHT, kSyrkStages>::LDS_BYTES <= (int)sizeof(smem), "stages fit");
    f64g_tile<RIGHT, kSyrkStages>(J.G, J.ldg, J.d, J.K, m0, n0, reinterpret_cast<unsigned char*>(smem), acc);
  } else {
    f64_tile<float, RIGHT, VEC, float, RIGHT, VEC>(J.G, J.ldg, J.G, J.ldg, J.d, J.d, J.K, m0, n0, smem, acc);
  }

  TS* S = reinterpret_cast<TS*>(J.S);
  const int64_t lds = J.lds;
  const int d = J.d;
  const double alpha = batch.alpha, beta = batch.beta;
  const bool packed = batch.packed != 0;
  f64_for_each(acc, [&](int r, int c, double v) {
    const int gr = m0 + r, gc = n0 + c;
    if (gr < d && gc < d && gr <= gc) {
      const int64_t i = sym_index(gr, gc, lds, d, packed);
      double val = alpha * v;
      if (beta != 0.0) val += beta * (double)S[i];
      const TS out = (TS)val;
      S[i] = out;
      if (!packed && gr != gc) S[(int64_t)gc * lds + gr] = out;
    }
  });
}

template <bool RIGHT, typename TS>
static hipError_t launch_syrk_t(const SyrkBatch& b, int vec, hipStream_t s) {
  if (vec == 4)
    hipLaunchKernelGGL((syrk_ema_kernel<RIGHT, TS, 4>), dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL((syrk_ema_kernel<RIGHT, TS, 1>), dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_syrk_ema(const SyrkBatch& b, bool right, bool f64_state, int vec, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (right) return f64_state ? launch_syrk_t<true, double>(b, vec, s) : launch_syrk_t<true, float>(b, vec, s);
  return f64_state ? launch_syrk_t<false, double>(b, vec, s) : launch_syrk_t<false, float>(b, vec, s);
}

}  // namespace mr
