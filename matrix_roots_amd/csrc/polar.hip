// O = U phi(Sigma / sqrt(L)) V^T for G = U Sigma V^T: ten CANS polar steps
// X <- a_k X + b_k X X^T X from X0 = G / sqrt(L), L = 1.01 ||G||_F^2
// (tilderesearch, "Online KL Shampoo", section 2.3; recurrence and layout in
// polar.hpp, coefficients and step bounds in cans.hpp).
//
// Per matrix: statistics (||G||_F^2, non-finite count) -> bound -> init
// (scaled G and G^T in split form) -> 20 GEMM launches for the whole batch ->
// finalize (O, and the residual ||A_9 - I||_F of the last Gram) -> info.
// Storage and products as in the inverse square root: split arrays (hi =
// fp16(x), lo = fp16((x - hi) 2^11)) times per-step powers of two, fp16
// (hi x hi) or split (three-product) MFMA, float32 accumulation.
#include <math.h>

#include <type_traits>

#include "epilogue.hpp"
#include "gemm_core.hpp"
#include "gemm_h16.hpp"
#include "polar.hpp"

namespace mr {

namespace {

struct Split {
  _Float16* hi;
  _Float16* lo;
  __device__ __forceinline__ SplitRef ref() const { return SplitRef{hi, lo}; }
};

// Buffer i of a matrix's region: 0, 1 = T for even / odd steps (M x N),
// 2 = T^T (N x M), 3 = A (N x N).
__device__ __forceinline__ Split polar_buf(char* region, int64_t M, int64_t N, int i) {
  const int64_t mn = M * N;
  const int64_t off = i < 3 ? (int64_t)i * 4 * mn : 12 * mn;
  const int64_t count = i < 3 ? mn : N * N;
  _Float16* h = reinterpret_cast<_Float16*>(region + off);
  return Split{h, h + count};
}

__device__ __forceinline__ void put(const Split& b, int64_t i, float v) {
  _Float16 h, l;
  split_f32(v, h, l);
  b.hi[i] = h;
  b.lo[i] = l;
}
__device__ __forceinline__ float get(const Split& b, int64_t i) { return join_f32(b.hi[i], b.lo[i]); }

__device__ __forceinline__ double block_sum(double v, double* red, int n) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int s = n / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int find_polar_job(const PolarBatch& B, int64_t b) {
  int jx = 0;
  while (jx + 1 < B.njobs && b >= B.job[jx + 1].block_begin) ++jx;
  return jx;
}

}  // namespace

// Per 8-row block of G: sum of squares and non-finite count.
__global__ __launch_bounds__(256) void polar_stats_kernel(const PolarBatch B) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const PolarJob& J = B.job[find_polar_job(B, b)];
  const int blk = (int)(b - J.block_begin);
  const int r0 = blk * kFinalRows, r1 = min(J.m, r0 + kFinalRows);
  double f2 = 0.0, nf = 0.0;
  for (int r = r0; r < r1; ++r)
    for (int c = threadIdx.x; c < J.n; c += 256) {
      const double v = (double)J.G[(int64_t)r * J.ldg + c];
      f2 += v * v;
      if (!isfinite(v)) nf += 1.0;
    }
  f2 = block_sum(f2, red, 256);
  nf = block_sum(nf, red, 256);
  if (threadIdx.x == 0) {
    double* p = B.partial + (int64_t)J.slot * B.partial_stride + 3 * blk;
    p[0] = 0.0;
    p[1] = f2;
    p[2] = nf;
    if (blk == 0) {
      RootState& st = B.state[J.slot];
      st.d = J.m;
      st.problem = J.problem;
      st.method = kCansMethod;
      st.eps = 0.0;
      st.sweeps = 0;
      st.residual = 0.f;
    }
  }
}

// One wave per matrix: s = ||G||_F^2 (fixed order), L = 1.01 s, flags.
__global__ __launch_bounds__(64) void polar_bound_kernel(RootState* state, const double* partial, int64_t stride,
                                                         int32_t nslots, double out_scale) {
  __shared__ double red[64];
  const int slot = blockIdx.x;
  if (slot >= nslots) return;
  RootState& st = state[slot];
  const int nb = (st.d + kFinalRows - 1) / kFinalRows;
  const double* p = partial + (int64_t)slot * stride;
  double f2 = 0.0, nf = 0.0;
  for (int i = threadIdx.x; i < nb; i += 64) {
    f2 += p[3 * i + 1];
    nf += p[3 * i + 2];
  }
  f2 = block_sum(f2, red, 64);
  nf = block_sum(nf, red, 64);
  if (threadIdx.x != 0) return;
  uint32_t flags = 0;
  int K = 0;
  if (nf > 0.0 || !isfinite(f2))
    flags = MR_INFO_NONFINITE;
  else if (f2 == 0.0)
    flags = MR_INFO_ZERO_TRACE;
  else
    K = kCansSteps;
  st.s = f2;
  st.c = kBoundSafety * f2;
  st.out_scale = out_scale;
  st.K = K;
  st.j = 0;
  st.flags = flags;
}

// s0 G / sqrt(L) into the m x n buffer and its transpose into the n x m one
// (T and T^T for a tall G, the other way round for a wide one), 32 x 32
// tiles through LDS so both writes are along rows.
__global__ __launch_bounds__(256) void polar_init_kernel(const PolarBatch B, double s0) {
  __shared__ double t[32][33];
  const int64_t b = blockIdx.x;
  const PolarJob& J = B.job[find_polar_job(B, b)];
  const RootState& st = B.state[J.slot];
  if (st.K == 0) return;
  const int m = J.m, n = J.n;
  const int tn = (n + 31) / 32;
  const int tile = (int)(b - J.block_begin);
  const int bi = tile / tn, bj = tile % tn;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bool tall = m >= n;
  const int64_t M = tall ? m : n, N = tall ? n : m;
  const Split GL = polar_buf(J.region, M, N, tall ? 0 : 2);  // m x n
  const Split GT = polar_buf(J.region, M, N, tall ? 2 : 0);  // n x m
  const double sc = s0 / sqrt(st.c);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = ty + 8 * e;
    const int gi = bi * 32 + r, gj = bj * 32 + tx;
    double v = 0.0;
    if (gi < m && gj < n) {
      v = sc * (double)J.G[(int64_t)gi * J.ldg + gj];
      put(GL, (int64_t)gi * n + gj, (float)v);
    }
    t[r][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = ty + 8 * e;
    const int gj = bj * 32 + r, gi = bi * 32 + tx;  // G^T[gj][gi] = G[gi][gj]
    if (gi < m && gj < n) put(GT, (int64_t)gj * m + gi, (float)t[tx][r]);
  }
}

// Stage A (FULL = false): A = alpha T^T T, upper tiles of N x N, mirrored.
// Stage X (FULL = true): T' = beta T + alpha T A, every tile of M x N,
// stored into T(k+1) and, transposed, into T^T.
// Block shapes: 128 x 128 for split products and for the fp16 Gram (whose
// few output tiles would leave the chip half idle with larger ones),
// kPolarTile-square tiles for the fp16 update.
constexpr int kPolarTile = 256;
constexpr int kPolarBK = 32;
using PolarSplitShape = H16Shape<128, 128, 2, 2>;
using PolarF16Shape = H16Shape<kPolarTile, kPolarTile, 2, kPolarTile / 64, kPolarBK>;

template <int VEC, int PREC, bool FULL, class S>
__global__ __launch_bounds__(S::THREADS, S::THREADS >= 512 ? 1 : 2) void polar_gemm_kernel(const PolarLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[PREC == 3 ? 2 * X3Tile::LDS_HALVES : h16_kernel_lds_bytes<S>(4 * kSlabFloats)];
  const int64_t b = blockIdx.x;
  int ci = 0;
  while (ci + 1 < L.ncls && b >= L.cls[ci + 1].block_begin) ++ci;
  const PolarClass& C = L.cls[ci];
  const int local = (int)xcd_remap(b - C.block_begin, round8(C.nblocks));
  if (local >= C.nblocks) return;
  const int mat = local / C.blocks_per_matrix;
  const int rem = local % C.blocks_per_matrix;
  if (L.state[C.slot_begin + mat].K == 0) return;
  const int M = C.M, N = C.N;
  char* region = C.region + (int64_t)mat * C.matrix_bytes;
  const int k = L.k;
  int ti, tj;
  Split Aop, Bop, Out;
  int rows, cols, K;
  int64_t lda, ldb;
  if (FULL) {
    full_tile_grouped(rem, C.TM, C.TN, ti, tj);
    Aop = polar_buf(region, M, N, k & 1);
    Bop = polar_buf(region, M, N, 3);
    Out = polar_buf(region, M, N, (k + 1) & 1);
    rows = M;
    cols = N;
    K = N;
    lda = N;
    ldb = N;
  } else {
    upper_tile_grouped(rem, C.TN, ti, tj);
    Aop = Bop = polar_buf(region, M, N, 2);
    Out = polar_buf(region, M, N, 3);
    rows = cols = N;
    K = M;
    lda = ldb = M;
  }
  const int m0 = ti * S::BM, n0 = tj * S::BN;
  v16f acc[S::RB][S::CB];
  if constexpr (PREC == 3)
    x3_nt_tile_auto<VEC>(Aop.ref(), lda, Bop.ref(), ldb, rows, cols, K, m0, n0, smem, acc);
  else
    h16_nt_tile_auto<S, VEC>(Aop.hi, lda, Bop.hi, ldb, rows, cols, K, m0, n0, smem, acc);
  // epilogue arithmetic: float64 for split products, float32 for fp16 ones
  using E = typename std::conditional<PREC == 3, double, float>::type;
  const E alpha = (E)L.alpha, beta = (E)L.beta;
  const Split Tt = polar_buf(region, M, N, 2);

  const bool whole = m0 + S::BM <= rows && n0 + S::BN <= cols;
  if (VEC == 8 && whole && (FULL || ti <= tj)) {
    // whole tile (update, or Gram on or above the diagonal): wide stores of
    // the tile and of its transpose (T^T, or the mirror) through per-wave LDS
    // slabs
    static_assert(S::CB == 2, "slab epilogue takes two 32-column blocks per wave");
    static_assert((S::THREADS / 64) * kSlabFloats * 4 <= (int)sizeof(smem), "one slab per wave fits in the LDS");
    const Split T = FULL ? Tt : Out;
    const int64_t ldt = FULL ? M : N;
    // fp16 products read X^T and A as operands only (hi halves); their lo
    // halves are kept for the last step (finalize and residual)
    const bool keep_lo = PREC == 3 || k == kCansSteps - 1;
    _Float16* out_lo = !FULL && !keep_lo ? nullptr : Out.lo;
    _Float16* t_lo = keep_lo ? T.lo : nullptr;
    wide_store_tile<S::RB, S::WN, E>(acc, reinterpret_cast<float*>(smem), m0, n0, Out.hi, out_lo, cols, T.hi, t_lo,
                                     ldt, FULL ? Aop.hi : nullptr, FULL ? Aop.lo : nullptr, alpha, beta, E(0),
                                     !FULL && ti == tj);
    return;
  }
  h16g_for_each<S>(acc, [&](int rr, int cc, float a) {
    const int gr = m0 + rr, gc = n0 + cc;
    if (gr >= rows || gc >= cols) return;
    if (FULL) {
      const int64_t i = (int64_t)gr * cols + gc;
      const float v = (float)(alpha * (E)a + beta * (E)get(Aop, i));
      put(Out, i, v);
      put(Tt, (int64_t)gc * M + gr, v);
    } else if (gr <= gc) {
      const float v = (float)(alpha * (E)a);
      put(Out, (int64_t)gr * cols + gc, v);
      if (gr != gc) put(Out, (int64_t)gc * cols + gr, v);
    }
  });
}

// O = out_scale * X_10 (m x n, the buffer holding that orientation), plus
// per-row-block partial sums of |A_9 - I|^2 over A's rows in the block.
// Flagged matrices: NaN (non-finite G) or zero (zero G).
__global__ __launch_bounds__(256) void polar_finalize_kernel(const PolarBatch B, double inv_sa9) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const PolarJob& J = B.job[find_polar_job(B, b)];
  const RootState& st = B.state[J.slot];
  const int m = J.m, n = J.n;
  const int blk = (int)(b - J.block_begin);
  const int r0 = blk * kFinalRows, r1 = min(m, r0 + kFinalRows);
  double res = 0.0;
  if (st.K == 0) {
    const float v = st.flags == MR_INFO_ZERO_TRACE ? 0.f : __builtin_nanf("");
    for (int r = r0; r < r1; ++r)
      for (int c = threadIdx.x; c < n; c += 256) J.O[(int64_t)r * J.ldo + c] = v;
  } else {
    const bool tall = m >= n;
    const int64_t M = tall ? m : n, N = tall ? n : m;
    const Split X = polar_buf(J.region, M, N, tall ? (kCansSteps & 1) : 2);  // m x n orientation of X_10
    const Split A = polar_buf(J.region, M, N, 3);
    const double sc = st.out_scale;
    for (int r = r0; r < r1; ++r)
      for (int c = threadIdx.x; c < n; c += 256)
        J.O[(int64_t)r * J.ldo + c] = (float)(sc * (double)get(X, (int64_t)r * n + c));
    for (int r = r0; r < min((int)N, r1); ++r)
      for (int c = threadIdx.x; c < N; c += 256) {
        const double e = (double)get(A, (int64_t)r * N + c) * inv_sa9 - (r == c ? 1.0 : 0.0);
        res += e * e;
      }
  }
  res = block_sum(res, red, 256);
  if (threadIdx.x == 0) B.partial[(int64_t)J.slot * B.partial_stride + blk] = res;
}

// ------------------------------------------------------------ launchers
hipError_t launch_polar_stats(const PolarBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(polar_stats_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_polar_bound(RootState* state, const double* partial, int64_t stride, int32_t nslots,
                              double out_scale, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  hipLaunchKernelGGL(polar_bound_kernel, dim3(nslots), dim3(64), 0, s, state, partial, stride, nslots, out_scale);
  return hipGetLastError();
}

hipError_t launch_polar_init(const PolarBatch& b, double s0, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(polar_init_kernel, dim3(b.total_blocks), dim3(256), 0, s, b, s0);
  return hipGetLastError();
}

int polar_tile(int prec, int stage) {
  return prec == 1 && stage == kPolarX ? PolarF16Shape::BM : PolarSplitShape::BM;
}

hipError_t launch_polar_gemm(const PolarLaunch& L, int vec, int prec, hipStream_t s) {
  if (L.total_blocks <= 0) return hipSuccess;
  const dim3 g(L.total_blocks);
  const bool full = L.stage == kPolarX;
#define MR_POLAR_LAUNCH(V, P, SH)                                                                       \
  do {                                                                                                  \
    if (full)                                                                                           \
      hipLaunchKernelGGL((polar_gemm_kernel<V, P, true, SH>), g, dim3(SH::THREADS), 0, s, L);          \
    else                                                                                                \
      hipLaunchKernelGGL((polar_gemm_kernel<V, P, false, SH>), g, dim3(SH::THREADS), 0, s, L);         \
  } while (0)
  if (prec == 3) {
    if (vec == 8)
      MR_POLAR_LAUNCH(8, 3, PolarSplitShape);
    else
      MR_POLAR_LAUNCH(1, 3, PolarSplitShape);
  } else {
    if (full) {
      if (vec == 8)
        MR_POLAR_LAUNCH(8, 1, PolarF16Shape);
      else
        MR_POLAR_LAUNCH(1, 1, PolarF16Shape);
    } else {
      if (vec == 8)
        MR_POLAR_LAUNCH(8, 1, PolarSplitShape);
      else
        MR_POLAR_LAUNCH(1, 1, PolarSplitShape);
    }
  }
#undef MR_POLAR_LAUNCH
  return hipGetLastError();
}

hipError_t launch_polar_finalize(const PolarBatch& b, double inv_sa9, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(polar_finalize_kernel, dim3(b.total_blocks), dim3(256), 0, s, b, inv_sa9);
  return hipGetLastError();
}

}  // namespace mr
