// Regularised inverse quarter root X = (A/s + eps I)^(-1/4) for Grams above
// the Jacobi size, by the GEMM-only coupled Newton iteration for the inverse
// p-th root with p = 4:
//
//   M0 = (A/s + eps I) / c,  X0 = I,
//   T_t = (5 I - M_t / s_t) / 4,  X_{t+1} = s_t^(-1/4) X_t T_t,
//   M_{t+1} = T_t^4 M_t / s_t,  X = c^(-1/4) X_K,
//
// with per-step scales s_t from the scalar schedule (schedule.hpp; s_t = 1
// is the classical iteration).
//
// The pages' step is "rescale, add a regulariser to the eigenvalues, raise to
// -1/4, rebuild" (marin.community, "Sharding EMA-Gram eigensolves", section
// "Background"); tilderesearch, "Online KL Shampoo", sections 2.1-2.2, argue
// for GEMM-only coupled iterations over eigendecompositions on GPUs and use
// the p = 2 member (coupled Newton-Schulz for S^(-1/2)) after normalising the
// largest eigenvalue below 1.  Every eigenvalue of M follows the scalar map
// m <- m ((5 - m)/4)^4, which is increasing on [0, 1] with fixed point 1, so
// the bounds of the spectrum, [eps/c, 1/1.01], fix the schedule.
//
// Per iteration: stage 0 computes T2 = T^2 = (25 I - 10 M/s + (M/s)^2)/16 and
// X' = s^(-1/4) (5 X - X M/s)/4 in one launch, stage 1 T4 = T2 T2, stage 2
// M' = T4 M / s.
// All matrices are polynomials in M0: symmetric and mutually commuting, so
// every product is an upper-tile symmetric GEMM.  The last iteration updates
// X only: the plain step, or a degree-2 or degree-4 Taylor finish in
// E = I - M (schedule.hpp).  M and its powers run in float64 while the
// schedule's floor of the spectrum of M is below kSwitchM, then on the
// split-fp16 kernels (float32-accurate products); X lives in split storage
// from the first step (the X update of a float64 step reads a split copy of
// M), or in float64 / float32 for MR_NEWTON_F64 / MR_NEWTON_F32.
//
// Buffers per matrix (region of 5 float64 slots of d*d, S0..S4, or 10
// half-slots h0..h9 of 4*d*d bytes): float64 M alternates S0/S3 (T2 the
// other), T4 is S4; a split matrix (hi[d*d] then lo[d*d]) fills a half-slot:
// M alternates h8/h0 (T2 the other), X h4/h2, T4 h9, the split copy of a
// float64 M h5, a degree-4 finish's q(M) h6.  Roles are a function of the
// iteration's parity, so every workgroup finds its operands without any
// table; the conversion at the switch writes the split M where the float64 M
// of that parity is not.
#include <math.h>

#include "epilogue.hpp"
#include "gemm_core.hpp"
#include "gemm_h16.hpp"
#include "gemm_i8.hpp"
#include "launch.hpp"
#include "schedule.hpp"

constexpr int kF64Occupancy = 2;  // workgroups per CU of the float64 Newton kernel
constexpr int kF32Occupancy = 2;  // ... and of the float32 one

namespace mr {

// ------------------------------------------------------------ roles
struct Roles64 {
  double *M, *T2, *X, *Xn, *T4;
};
struct Roles32 {
  float *M, *T2, *X, *Xn, *T4;
};
__host__ __device__ __forceinline__ Roles64 roles64(char* region, int d, int t) {
  const int64_t S = (int64_t)d * d * 8;
  const bool even = (t & 1) == 0;
  Roles64 r;
  r.M = reinterpret_cast<double*>(region + (even ? 0 : 3) * S);
  r.T2 = reinterpret_cast<double*>(region + (even ? 3 : 0) * S);
  r.X = reinterpret_cast<double*>(region + (even ? 1 : 2) * S);
  r.Xn = reinterpret_cast<double*>(region + (even ? 2 : 1) * S);
  r.T4 = reinterpret_cast<double*>(region + 4 * S);
  return r;
}
__device__ __forceinline__ Roles32 roles32(char* region, int d, int t) {
  const int64_t H = (int64_t)d * d * 4;
  const bool even = (t & 1) == 0;
  Roles32 r;
  r.M = reinterpret_cast<float*>(region + (even ? 8 : 0) * H);
  r.T2 = reinterpret_cast<float*>(region + (even ? 0 : 8) * H);
  r.X = reinterpret_cast<float*>(region + (even ? 4 : 2) * H);
  r.Xn = reinterpret_cast<float*>(region + (even ? 2 : 4) * H);
  r.T4 = reinterpret_cast<float*>(region + 9 * H);
  return r;
}

// Split storage (default Newton path): a half-slot h holds hi[d*d] then
// lo[d*d] (fp16 each), value = hi + 2^-11 lo.  Float32 steps use the Roles32
// positions; during float64 steps X sits at its Roles32 position too and the
// split copy of the float64 M for the X update (Mx) at half-slot 5.
struct SplitBuf {
  _Float16* hi;
  _Float16* lo;
  __device__ SplitRef ref() const { return SplitRef{hi, lo}; }
};
__host__ __device__ __forceinline__ SplitBuf split_at(char* region, int d, int h) {
  _Float16* hi = reinterpret_cast<_Float16*>(region + (int64_t)h * d * d * 4);
  return SplitBuf{hi, hi + (int64_t)d * d};
}
struct RolesS {
  SplitBuf M, T2, X, Xn, T4, Mx, Q;
};
__host__ __device__ __forceinline__ RolesS roless(char* region, int d, int t) {
  const bool even = (t & 1) == 0;
  RolesS r;
  r.M = split_at(region, d, even ? 8 : 0);
  r.T2 = split_at(region, d, even ? 0 : 8);
  r.X = split_at(region, d, even ? 4 : 2);
  r.Xn = split_at(region, d, even ? 2 : 4);
  r.T4 = split_at(region, d, 9);
  r.Mx = split_at(region, d, 5);
  r.Q = split_at(region, d, 6);  // the degree-4 finish's q(M) (a float64 slot, dead in split steps)
  return r;
}
// X is stored times 2^-e so that |X| <= (eps/c)^(-1/4) stays below 2^13 in
// fp16 (X updates are linear in X; the finalize undoes the scale).
__device__ __forceinline__ float x_store_scale(const RootState& st) {
  const double xmax = pow(st.eps / st.c, -0.25);
  const int e = (int)ceil(log2(xmax)) - 13;
  return e > 0 ? ldexpf(1.0f, -e) : 1.0f;
}
__device__ __forceinline__ void split_put(const SplitBuf& b, int64_t i, float v) {
  _Float16 h, l;
  split_f32(v, h, l);
  b.hi[i] = h;
  b.lo[i] = l;
}

// ------------------------------------------------------ block reductions
// Fixed-order tree over 256 threads: the same inputs give the same bits.
__device__ __forceinline__ double block_sum_256(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
__device__ __forceinline__ double block_sum_64(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 32; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int find_job(const RootBatch& B, int64_t b) {
  int jx = 0;
  while (jx + 1 < B.njobs && b >= B.job[jx + 1].block_begin) ++jx;
  return jx;
}

template <typename TA>
__device__ __forceinline__ double ld_elem(const void* A, int64_t idx) {
  return (double)reinterpret_cast<const TA*>(A)[idx];
}

// ------------------------------------------------------------ statistics
// Per 32-row stripe of A: partial trace, sum of squares, count of
// non-finite, over 32 x 32 tiles left to right, each thread summing its own
// tile positions in that order.  A packed A's lower tiles are their upper
// mirrors transposed through LDS, so a packed and a full copy of the same
// symmetric matrix give bitwise identical partials.
template <typename TA>
__global__ __launch_bounds__(256) void root_stats_kernel(const RootBatch B) {
  __shared__ double red[256];
  __shared__ double tl[32][33];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_job(B, b)];
  const int blk = (int)(b - J.block_begin);
  const int d = J.d;
  const int T = (d + 31) / 32;
  const bool packed = B.a_packed != 0;
  const TA* A = reinterpret_cast<const TA*>(J.A);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  double tr = 0.0, f2 = 0.0, nf = 0.0;
  for (int bj = 0; bj < T; ++bj) {
    const bool mirror = packed && bj < blk;
    if (mirror) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = ty + 8 * e;
        const int gi = bj * 32 + r, gj = blk * 32 + tx;
        tl[r][tx] = (gi < d && gj < d) ? (double)A[sym_index(gi, gj, 0, d, true)] : 0.0;
      }
      __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = ty + 8 * e;
      const int gi = blk * 32 + r, gj = bj * 32 + tx;
      if (gi < d && gj < d) {
        const double v = mirror ? tl[tx][r] : (double)A[sym_index(gi, gj, J.lda, d, packed)];
        if (gi == gj) tr += v;
        f2 += v * v;
        if (!isfinite(v)) nf += 1.0;
      }
    }
  }
  tr = block_sum_256(tr, red);
  f2 = block_sum_256(f2, red);
  nf = block_sum_256(nf, red);
  if (threadIdx.x == 0) {
    double* p = B.partial + (int64_t)J.slot * B.partial_stride + 3 * blk;
    p[0] = tr;
    p[1] = f2;
    p[2] = nf;
    if (blk == 0) {
      RootState& st = B.state[J.slot];
      st.d = d;
      st.problem = J.problem;
      st.method = MR_NEWTON;
      st.eps = B.eps;
      st.sweeps = 0;
      st.residual = 0.f;
    }
  }
}

// One wave per matrix: combine the partials in a fixed order, then derive
// s, the bound c, the iteration count K and the switch iteration j.
//
// c = 1.01 * WS(A/s + eps I), where WS(B) = m + sqrt(max(|B|_F^2/d - m^2, 0)) *
// sqrt(d - 1), m = tr(B)/d, is the Wolkowicz-Styan upper bound on the largest
// eigenvalue of a symmetric matrix (the OKLS page, appendix D, bounds the
// largest eigenvalue by the minimum of this and a second bound before its
// iteration).  |A|_F is taken over A itself, which bounds that of (A + A^T)/2.
// For a positive semidefinite A/s of unit trace WS <= 1 + eps.
__global__ __launch_bounds__(64) void root_bound_kernel(RootState* state, double* partial,
                                                        int64_t stride, double* sched, int32_t slot_begin,
                                                        int32_t normalize, double eps, int32_t k_cap,
                                                        double floor_cap, int32_t all_f64, int32_t finish) {
  __shared__ double red[64];
  const int slot = slot_begin + blockIdx.x;
  RootState& st = state[slot];
  const int d = st.d;
  const int nb = (d + kStatsRows - 1) / kStatsRows;
  const double* p = partial + (int64_t)slot * stride;
  double tr = 0.0, f2 = 0.0, nf = 0.0;
  for (int i = threadIdx.x; i < nb; i += 64) {
    tr += p[3 * i + 0];
    f2 += p[3 * i + 1];
    nf += p[3 * i + 2];
  }
  tr = block_sum_64(tr, red);
  f2 = block_sum_64(f2, red);
  nf = block_sum_64(nf, red);
  if (threadIdx.x != 0) return;
  uint32_t flags = 0;
  double s = 1.0, c = 1.0;
  int K = 0, j = 0, fin = 1;
  if (nf > 0.0 || !isfinite(tr) || !isfinite(f2)) {
    flags |= MR_INFO_NONFINITE;
  } else {
    if (normalize == MR_NORM_TRACE) s = tr;
    if (normalize == MR_NORM_TRACE && s == 0.0) {
      flags |= MR_INFO_ZERO_TRACE;
    } else {
      const double trh = tr / s;
      const double f2h = f2 / (s * s);
      const double dd = (double)d;
      const double trB = trh + dd * eps;
      const double f2B = f2h + 2.0 * eps * trh + dd * eps * eps;
      const double m = trB / dd;
      const double var = fmax(f2B / dd - m * m, 0.0);
      const double ws = m + sqrt(var) * sqrt(dd - 1.0);
      c = kBoundSafety * ws;
      if (!(c > 0.0) || !isfinite(c)) {
        flags |= MR_INFO_NOT_PD;
        c = 1.0;
      } else {
        // |B/c|_F^2 for the fourth-moment bound (the stripe partials are read)
        partial[(int64_t)slot * stride + 1] = f2B / (c * c);
        // The host launches the schedule of floor_cap: a matrix whose floor
        // lies lower runs exactly that schedule (its steps and its float64
        // steps are then those the host launches; both counts only fall as
        // the floor rises) and is not iterated to convergence, and says so.
        double floor = fmin(eps / c, 1.0 / kBoundSafety);
        if (floor < floor_cap) {
          floor = floor_cap;
          flags |= MR_INFO_NOT_CONVERGED;
        }
        newton_scaled_schedule(floor, 1.0 / kBoundSafety, kNewtonTol, kSwitchM, k_cap,
                               sched + (int64_t)slot * kMaxNewtonIters, &K, &j, finish != 0, &fin);
        if (all_f64) j = K;
      }
    }
  }
  st.s = s;
  st.c = c;
  st.out_scale = pow(c, -0.25);
  st.K = K;
  st.j = j;
  st.fin = fin;
  st.flags = flags;
}

// ------------------------------------------------------------ fourth-moment bound
// A second upper bound on the largest eigenvalue beside Wolkowicz-Styan (the
// OKLS page, appendix D, takes the smaller of two bounds in the same place):
// for a symmetric H, |mu|_max(H)^4 <= tr(H^4) = |H^2|_F^2.  H is the fp16 copy
// of B/c (B = A/s + eps I, c the Wolkowicz-Styan bound), its square comes from
// fp16 products with float32 sums, and the tighten kernel adds the rounding of
// both to the bound (Weyl's inequality for the copy, the float32 sum error
// for the product), so the result stays an upper bound.  On Grams of gradients
// it is 2-3 times tighter than Wolkowicz-Styan: a higher floor eps/c, fewer
// Newton steps.

// H = fp16((A/s + eps I)/c), zero-padded to dp = moment_pad(d), row stride dp,
// at the start of the matrix's region (root_init writes M0 there afterwards):
// the 32 x 32 tile pairs of root_init over the padded grid.
template <typename TA>
__global__ __launch_bounds__(256) void root_moment_convert_kernel(const RootBatch B) {
  __shared__ double ta[32][33];
  __shared__ double tb[32][33];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_job(B, b)];
  const RootState& st = B.state[J.slot];
  const int d = J.d;
  if (st.K == 0 || d < kMomentMinD) return;
  const int dp = moment_pad(d);
  int bi, bj;
  upper_pair((int)(b - J.block_begin), dp / 32, bi, bj);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bool packed = B.a_packed != 0;
  load_sym_tile<TA>(J.A, J.lda, d, packed, bi, bj, ta, tb);  // zero past d
  const double inv_s = 1.0 / st.s, inv_c = 1.0 / st.c, eps = B.eps;
  _Float16* H = reinterpret_cast<_Float16*>(J.region);
  auto put = [&](int gi, int gj, double sym) __attribute__((always_inline)) {
    const double v = gi < d && gj < d ? (sym * inv_s + (gi == gj ? eps : 0.0)) * inv_c : 0.0;
    H[(int64_t)gi * dp + gj] = (_Float16)v;
  };
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = ty + 8 * e;
    put(bi * 32 + r, bj * 32 + tx, sym_tile_value(packed, bi, bj, r, tx, ta, tb));
    if (bi != bj) put(bj * 32 + r, bi * 32 + tx, sym_tile_value(packed, bi, bj, tx, r, ta, tb));
  }
}

// Pass 0: sum of squares of the upper 128 x 128 tile u of P = H H (twice for
// tiles off the diagonal), elements past d left out, into partial[2 + u] of
// the matrix, and the tile and its mirror as fp16 into P16 (dp x dp after
// H in the region).  Pass 1: the same sums for P16 P16 into partial[2 + U + u].
using MomentShape = H16Shape<kMomentTile, kMomentTile, 2, 2>;
static_assert(MomentShape::THREADS == 256, "block_sum_256");
template <int PASS>
__global__ __launch_bounds__(256) void root_moment_kernel(const RootBatch B) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[h16_lds_bytes<MomentShape>()];
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_job(B, b)];
  const RootState& st = B.state[J.slot];
  const int d = J.d;
  if (st.K == 0 || d < kMomentMinD) return;
  const int dp = moment_pad(d);
  const int T = (dp + kMomentTile - 1) / kMomentTile;
  const int u = (int)(b - J.block_begin);
  int ti, tj;
  upper_pair(u, T, ti, tj);
  _Float16* H = reinterpret_cast<_Float16*>(J.region);
  _Float16* P16 = H + (int64_t)dp * dp;
  const _Float16* In = PASS == 0 ? H : P16;
  v16f acc[MomentShape::RB][MomentShape::CB];
  // dp is a multiple of 64: the direct-to-LDS core, whole 64-deep chunks
  h16_nt_tile_auto<MomentShape, 8>(In, dp, In, dp, dp, dp, dp, ti * kMomentTile, tj * kMomentTile, smem, acc);
  double sq = 0.0;
  h16g_for_each<MomentShape>(acc, [&](int rr, int cc, float v) {
    const int gr = ti * kMomentTile + rr, gc = tj * kMomentTile + cc;
    if (gr < d && gc < d) sq += (double)v * (double)v;
    if (PASS == 0 && gr < dp && gc < dp && (ti != tj || rr <= cc)) {  // one writer per pair: P16 symmetric
      P16[(int64_t)gr * dp + gc] = (_Float16)v;
      P16[(int64_t)gc * dp + gr] = (_Float16)v;
    }
  });
  sq = block_sum_256(sq, red);
  if (threadIdx.x == 0)
    B.partial[(int64_t)J.slot * B.partial_stride + 2 + PASS * moment_tiles(d) + u] = (ti == tj ? 1.0 : 2.0) * sq;
}

// One wave per matrix: the fourth-moment bound from the tile sums, and where
// it is below the Wolkowicz-Styan c, that c and its schedule instead.
//   |H^2|_F <= |P|_F + g |H|_F^2, g = d u / (1 - d u), u = 2^-24 (float32 sums
//     of exact fp16 products, in any order),
//   lambda_max(B/c) <= |mu|_max(H) + |B/c - H|_F, |B/c - H|_F <= 2^-11 |B/c|_F
//     + d 2^-25 (fp16 rounding: half an ulp, or half the smallest subnormal),
// |H|_F <= (1 + 2^-11) |B/c|_F + d 2^-25.
__global__ __launch_bounds__(64) void root_tighten_kernel(RootState* state, const double* partial, int64_t stride,
                                                          double* sched, int32_t slot_begin, double eps,
                                                          int32_t k_cap, double floor_cap, int32_t all_f64,
                                                          int32_t finish) {
  __shared__ double red[64];
  const int slot = slot_begin + blockIdx.x;
  RootState& st = state[slot];
  if (st.K == 0 || st.d < kMomentMinD) return;
  const double* p = partial + (int64_t)slot * stride;
  const int U = moment_tiles(st.d);
  double m4 = 0.0, m8 = 0.0;
  for (int i = threadIdx.x; i < U; i += 64) {
    m4 += p[2 + i];
    m8 += p[2 + U + i];
  }
  m4 = block_sum_64(m4, red);
  m8 = block_sum_64(m8, red);
  if (threadIdx.x != 0) return;
  const double dd = (double)moment_pad(st.d);
  const double fb = sqrt(p[1]);  // |B/c|_F
  const double nh = (1.0 + 0x1p-11) * fb + dd * 0x1p-25;
  const double g = dd * 0x1p-24 / (1.0 - dd * 0x1p-24);
  // fourth moment: |mu|_max(H)^2 <= |H^2|_F <= |P|_F + g |H|_F^2
  const double e2 = g * nh * nh;  // |P - H^2|_F
  const double mu4 = sqrt(sqrt(m4) + e2);
  // eighth moment through P16 = fp16(P), symmetric: |mu|_max(H)^2 =
  // |nu|_max(H^2) <= |nu|_max(P16) + |P16 - H^2|_F, |nu|_max(P16)^2 <=
  // |P16^2|_F <= |Q|_F + g |P16|_F^2 (Q the float32 product of P16)
  const double np = sqrt(m4);  // |P|_F
  const double np16 = (1.0 + 0x1p-11) * np + dd * 0x1p-25;
  const double nu = sqrt(sqrt(m8) + g * np16 * np16) + 0x1p-11 * np + dd * 0x1p-25 + e2;
  const double mu8 = sqrt(nu);
  const double beta = fmin(mu4, mu8) + 0x1p-11 * fb + dd * 0x1p-25;
  const double c = kBoundSafety * st.c * beta;
  if (!(c > 0.0) || !(c < st.c) || !isfinite(c)) return;
  double floor = fmin(eps / c, 1.0 / kBoundSafety);
  uint32_t flags = st.flags & ~(uint32_t)MR_INFO_NOT_CONVERGED;
  if (floor < floor_cap) {
    floor = floor_cap;
    flags |= MR_INFO_NOT_CONVERGED;
  }
  int K = 0, j = 0, fin = 1;
  newton_scaled_schedule(floor, 1.0 / kBoundSafety, kNewtonTol, kSwitchM, k_cap,
                         sched + (int64_t)slot * kMaxNewtonIters, &K, &j, finish != 0, &fin);
  if (all_f64) j = K;
  st.c = c;
  st.out_scale = pow(c, -0.25);
  st.K = K;
  st.j = j;
  st.fin = fin;
  st.flags = flags;
}


// M0 = ((A + A^T)/2 / s + eps I) / c into S0 (float64), one workgroup per
// pair of mirrored 32 x 32 tiles (upper_pair), both read once through LDS so
// every A read and write is coalesced.  X: with split storage the
// first X update needs no product (X0 = I, so X1 = s0^(-1/4) (5 I - M0/s0) / 4)
// and is written here, in the buffer iteration 1 reads; otherwise X0 = I
// into S1 (float64) for the first step's product.
template <typename TA>
__global__ __launch_bounds__(256) void root_init_kernel(const RootBatch B) {
  __shared__ double ta[32][33];
  __shared__ double tb[32][33];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_job(B, b)];
  const RootState& st = B.state[J.slot];
  if (st.K == 0) return;
  const int d = J.d;
  const int Tt = (d + 31) / 32;
  int bi, bj;
  upper_pair((int)(b - J.block_begin), Tt, bi, bj);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bool packed = B.a_packed != 0;
  load_sym_tile<TA>(J.A, J.lda, d, packed, bi, bj, ta, tb);
  const double inv_s = 1.0 / st.s, inv_c = 1.0 / st.c, eps = B.eps;
  double* M = reinterpret_cast<double*>(J.region);
  double* X = reinterpret_cast<double*>(J.region + (int64_t)d * d * 8);
  const RolesS rs = roless(J.region, d, 0);
  const SplitBuf x1 = roless(J.region, d, 1).X;
  const float xs = B.x_low ? x_store_scale(st) : 1.0f;
  const double s0 = B.x_low ? B.sched[(int64_t)J.slot * kMaxNewtonIters] : 1.0;
  const double q0 = (double)xs * pow(s0, -0.25), inv_s0 = 1.0 / s0;
  auto put = [&](int gi, int gj, double sym) __attribute__((always_inline)) {
    const double v = (sym * inv_s + (gi == gj ? eps : 0.0)) * inv_c;
    const int64_t e = (int64_t)gi * d + gj;
    M[e] = v;
    if (B.x_low) {
      split_put(rs.Mx, e, (float)v);
      split_put(x1, e, (float)(q0 * ((gi == gj ? 1.25 : 0.0) - 0.25 * v * inv_s0)));
    } else {
      X[e] = (gi == gj) ? 1.0 : 0.0;
    }
  };
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = ty + 8 * e;
    // tile (bi, bj), then its mirror (bj, bi) from the same LDS tiles
    if (bi * 32 + r < d && bj * 32 + tx < d) put(bi * 32 + r, bj * 32 + tx, sym_tile_value(packed, bi, bj, r, tx, ta, tb));
    if (bi != bj && bj * 32 + r < d && bi * 32 + tx < d)
      put(bj * 32 + r, bi * 32 + tx, sym_tile_value(packed, bi, bj, tx, r, ta, tb));
  }
}

// ------------------------------------------------------------ Newton GEMMs
__device__ __forceinline__ int find_class(const NewtonLaunch& L, int64_t b) {
  int ci = 0;
  while (ci + 1 < L.ncls && b >= L.cls[ci + 1].block_begin) ++ci;
  return ci;
}

struct StageJob {
  bool active;
  int job;
  int fin;  // this iteration's finish degree (1: a plain step)
  int ti, tj;
  int d;
  char* region;
  double s;   // step scale
  double m0;  // floor of the initial spectrum, eps / c
};

// Which kernel runs a (matrix, stage, job) at iteration t:
//   kStageF64  : t < j (float64 steps); with x_low not the X update
//   kStageX3B64: t < j, X update only (x_low: float32 X, float64 M)
//   kStageF32 / kStageX3: t >= j (float32 steps)
// and the last iteration (t = K-1) only updates X (stage 0, job 1); with
// x_low the first X update (t = 0) was written by root_init_kernel.
__device__ __forceinline__ StageJob stage_job(const NewtonLaunch& L, int kind) {
  StageJob s;
  const int64_t b = blockIdx.x;
  const NewtonClass& C = L.cls[find_class(L, b)];
  const int local = (int)xcd_remap(b - C.block_begin, round8(C.nblocks));
  if (local >= C.nblocks) {
    s.active = false;
    return s;
  }
  const int mat = local / C.blocks_per_matrix;
  const int rem = local % C.blocks_per_matrix;
  s.job = L.job_only >= 0 ? L.job_only : rem / C.U;
  upper_tile_grouped(rem % C.U, C.T, s.ti, s.tj);
  s.d = C.d;
  s.region = C.region + (int64_t)mat * C.matrix_bytes;
  const int slot = C.slot_begin + mat;
  const RootState& st = L.state[slot];
  const int t = L.t, K = st.K, j = st.j;
  const bool xupdate = L.stage == 0 && s.job == 1;
  bool act;
  if (kind == kStageF64 || kind == kStageI8)
    act = t < K && t < j && !(L.x_low && xupdate);
  else if (kind == kStageX3B64)
    act = t < K && t < j && L.x_low && xupdate;
  else
    act = t >= j && t < K;
  if (t == K - 1) {
    if (st.fin <= 1) {
      if (!xupdate) act = false;
    } else {
      // Taylor finish (split steps): job 0 of stages 0..1 (degree 2) or 0..2 (degree 4)
      act = act && s.job == 0 && L.stage <= (st.fin == 2 ? 1 : 2);
    }
  }
  if (t == 0 && xupdate && L.x_low) act = false;
  s.fin = t == K - 1 ? st.fin : 1;
  s.active = act;
  s.s = act ? L.sched[(int64_t)slot * kMaxNewtonIters + t] : 1.0;
  s.m0 = st.eps / st.c;
  return s;
}

template <typename T>
struct StageOps {
  const T *A, *B, *Cin;
  T* C;
  double alpha, beta, gamma;
};

template <typename T, typename R>
__device__ __forceinline__ StageOps<T> stage_ops(const R& r, int stage, int job, double s) {
  StageOps<T> o;
  o.Cin = nullptr;
  o.beta = 0.0;
  o.gamma = 0.0;
  o.alpha = 1.0;
  const double is = 1.0 / s;
  if (stage == 0 && job == 0) {  // T2 = ((M/s)^2 - 10 M/s + 25 I) / 16
    o.A = r.M; o.B = r.M; o.C = r.T2; o.Cin = r.M;
    o.alpha = is * is / 16.0; o.beta = -10.0 * is / 16.0; o.gamma = 25.0 / 16.0;
  } else if (stage == 0) {  // X' = s^(-1/4) (5 X - X M/s) / 4
    const double q = pow(s, -0.25);
    o.A = r.X; o.B = r.M; o.C = r.Xn; o.Cin = r.X;
    o.alpha = -0.25 * q * is; o.beta = 1.25 * q;
  } else if (stage == 1) {  // T4 = T2 T2
    o.A = r.T2; o.B = r.T2; o.C = r.T4;
  } else {  // M' = T4 M / s, written over T2 (dead after stage 1)
    o.A = r.T4; o.B = r.M; o.C = r.T2;
    o.alpha = is;
  }
  return o;
}

template <typename T>
__device__ __forceinline__ void sym_store(const StageOps<T>& o, int d, int gr, int gc, double v) {
  if (gr < d && gc < d && gr <= gc) {
    double val = o.alpha * v;
    if (o.Cin) val += o.beta * (double)o.Cin[(int64_t)gr * d + gc];
    if (gr == gc) val += o.gamma;
    const T out = (T)val;
    o.C[(int64_t)gr * d + gc] = out;
    if (gr != gc) o.C[(int64_t)gc * d + gr] = out;
  }
}

// Float64 epilogue of a whole 128 x 128 tile (d even).  A lane of a 16 x 16
// float64 MFMA block holds one column and four rows, so the upper elements go
// straight from the accumulators (16 lanes write 128 consecutive bytes of a
// row), while their mirror would be 8-byte stores d * 8 bytes apart.  Each
// wave therefore also puts its values, 32 rows at a time, into a private LDS
// slab and writes columns of it as rows of the mirror, 8 values (64 bytes) per
// lane.  plain: C = alpha acc (stage 2 of a float64 step, which also writes the
// split copy mx of C); else C = alpha acc + beta Cin (+ gamma on the
// diagonal), the values of sym_store.  diag: a tile on the diagonal (r <= c
// stored, r < c mirrored).  The main loop ended with a block barrier, so the
// operand stages are free.
constexpr int kF64SlabLd = 64 + 2;  // doubles per slab row
__device__ __forceinline__ void f64_store_tile(const v4d (&acc)[4][4], double* lds, int d, int m0, int n0,
                                               const StageOps<double>& o, bool plain, const SplitBuf& mx, bool diag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  double* slab = lds + wave * 32 * kF64SlabLd;
  const bool mx_vec = d % 8 == 0;  // 16-byte split stores of 8 halves
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int lr = rb2 * 16 + f64_row(lane, v), lc = cb * 16 + (lane & 15);
          const int gr = m0 + wm * 64 + h * 32 + lr, gc = n0 + wn * 64 + lc;
          const int64_t e = (int64_t)gr * d + gc;
          double val = o.alpha * acc[2 * h + rb2][cb][v];
          if (!plain) {
            if (o.Cin) val += o.beta * o.Cin[e];
            if (gr == gc) val += o.gamma;
          }
          if (!diag || gr <= gc) {
            o.C[e] = val;
            if (plain) split_put(mx, e, (float)val);
          }
          slab[lr * kF64SlabLd + lc] = val;
        }
    slab_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane + 64 * i;
      const int c = q >> 2, rg = q & 3;  // slab column, group of 8 rows
      const int gc = n0 + wn * 64 + c, gr0 = m0 + wm * 64 + h * 32 + rg * 8;
      if (diag && gr0 >= gc) continue;  // no element of the group above the diagonal
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = slab[(rg * 8 + e) * kF64SlabLd + c];
      const int64_t t = (int64_t)gc * d + gr0;  // mirror: C[gc][gr0 + e] = value at (gr0 + e, gc)
      if (!diag || gr0 + 7 < gc) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) *reinterpret_cast<v2d*>(o.C + t + e) = v2d{v[e], v[e + 1]};
        if (plain) {
          if (mx_vec) {
            v8h hh, ll;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              _Float16 a, b;
              split_f32((float)v[e], a, b);
              hh[e] = a;
              ll[e] = b;
            }
            *reinterpret_cast<v8h*>(mx.hi + t) = hh;
            *reinterpret_cast<v8h*>(mx.lo + t) = ll;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) split_put(mx, t + e, (float)v[e]);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gr0 + e < gc) {
            o.C[t + e] = v[e];
            if (plain) split_put(mx, t + e, (float)v[e]);
          }
      }
    }
    slab_fence();
  }
}

template <int VEC>
__global__ __launch_bounds__(256, VEC == 2 ? kF64Occupancy : 1) void newton_f64_kernel(const NewtonLaunch L) {
  // (with x_low, stage 2 also writes the split copy Mx of the new M)
  __shared__ __attribute__((aligned(16))) double smem[F64Tile::LDS_DOUBLES];
  static_assert(4 * 32 * kF64SlabLd <= F64Tile::LDS_DOUBLES, "four 32-row slabs fit in the operand stages");
  const StageJob s = stage_job(L, kStageF64);
  if (!s.active) return;
  const Roles64 r = roles64(s.region, s.d, L.t);
  const StageOps<double> o = stage_ops<double>(r, L.stage, s.job, s.s);
  const int m0 = s.ti * F64Tile::BM, n0 = s.tj * F64Tile::BN;
  v4d acc[4][4];
  f64_nt_tile_auto<VEC>(o.A, s.d, o.B, s.d, s.d, s.d, s.d, m0, n0, smem, acc);
  const int d = s.d;
  const bool plain = L.x_low && L.stage == 2;
  const SplitBuf mx = roless(s.region, d, L.t).Mx;
  // (Grams below 256 keep the element stores: their tiles are latency-bound,
  // and the slab passes cost more than the scattered mirror stores there)
  if (VEC == 2 && d >= 256 && m0 + F64Tile::BM <= d && n0 + F64Tile::BN <= d) {
    f64_store_tile(acc, smem, d, m0, n0, o, plain, mx, s.ti == s.tj);
  } else if (plain) {
    f64_for_each(acc, [&](int rr, int cc, double v) {
      const int gr = m0 + rr, gc = n0 + cc;
      if (gr < d && gc < d && gr <= gc) {
        const double val = o.alpha * v;
        o.C[(int64_t)gr * d + gc] = val;
        split_put(mx, (int64_t)gr * d + gc, (float)val);
        if (gr != gc) {
          o.C[(int64_t)gc * d + gr] = val;
          split_put(mx, (int64_t)gc * d + gr, (float)val);
        }
      }
    });
  } else {
    f64_for_each(acc, [&](int rr, int cc, double v) { sym_store(o, d, m0 + rr, n0 + cc, v); });
  }
}

template <int VEC>
__global__ __launch_bounds__(256, kF32Occupancy) void newton_f32_kernel(const NewtonLaunch L) {
  __shared__ float smem[F32Tile::LDS_FLOATS];
  const StageJob s = stage_job(L, kStageF32);
  if (!s.active) return;
  const Roles32 r = roles32(s.region, s.d, L.t);
  const StageOps<float> o = stage_ops<float>(r, L.stage, s.job, s.s);
  const int m0 = s.ti * F32Tile::BM, n0 = s.tj * F32Tile::BN;
  v16f acc[2][2];
  f32_nt_tile<VEC>(o.A, s.d, o.B, s.d, s.d, s.d, s.d, m0, n0, smem, acc);
  const int d = s.d;
  f32_for_each(acc, [&](int rr, int cc, float v) { sym_store(o, d, m0 + rr, n0 + cc, (double)v); });
}

// Float32 steps on the fp16 matrix cores with split storage (see
// x3_nt_tile).  kStageX3B64: the X update of a float64 step, X times the
// split copy Mx of the float64 M -- M enters X' = s^(-1/4)(5X - XM/s)/4 only
// as a perturbation of 5, so its float32 rounding is harmless there.
struct SplitOps {
  SplitRef A, B, Cin;
  SplitBuf C, C2;  // C2: a second output of the same product (degree-4 finish)
  bool has_cin, has_c2;
  double alpha, beta, gamma;
  double alpha2, beta2, gamma2;
};

// Coefficients of the Taylor series of (1 - x)^(-1/4): c_k = c_{k-1} (k - 3/4) / k.
constexpr double kTay0 = 1.0, kTay1 = 0.25, kTay2 = 5.0 / 32.0, kTay3 = 15.0 / 128.0, kTay4 = 195.0 / 2048.0;

__device__ __forceinline__ SplitOps split_ops(const RolesS& r, int stage, int job, double s, bool xm, int fin = 1) {
  SplitOps o;
  o.has_cin = false;
  o.has_c2 = false;
  o.alpha = 1.0;
  o.beta = 0.0;
  o.gamma = 0.0;
  const double is = 1.0 / s;
  if (fin == 2) {  // last step, degree-2 Taylor finish in E = I - M
    if (stage == 0) {  // Q = c0 + c1 E + c2 E^2 = c2 M^2 - (c1 + 2 c2) M + (c0 + c1 + c2) I
      o.A = r.M.ref(); o.B = r.M.ref(); o.C = r.T2; o.Cin = r.M.ref(); o.has_cin = true;
      o.alpha = kTay2; o.beta = -(kTay1 + 2.0 * kTay2); o.gamma = kTay0 + kTay1 + kTay2;
    } else {  // X' = X Q
      o.A = r.X.ref(); o.B = r.T2.ref(); o.C = r.Xn;
    }
    return o;
  }
  if (fin == 4) {  // last step, degree-4 Taylor finish: q = c0 + c1 E + E^2 (c2 + c3 E + c4 E^2)
    if (stage == 0) {  // E^2 = M^2 - 2M + I, and R = c2 + c3 E + c4 E^2 from the same M^2
      o.A = r.M.ref(); o.B = r.M.ref(); o.C = r.T2; o.Cin = r.M.ref(); o.has_cin = true;
      o.alpha = 1.0; o.beta = -2.0; o.gamma = 1.0;
      o.C2 = r.T4; o.has_c2 = true;
      o.alpha2 = kTay4; o.beta2 = -(2.0 * kTay4 + kTay3); o.gamma2 = kTay2 + kTay3 + kTay4;
    } else if (stage == 1) {  // Q = E^2 R + c1 E + c0 I = E^2 R - c1 M + (c0 + c1) I
      o.A = r.T2.ref(); o.B = r.T4.ref(); o.C = r.Q; o.Cin = r.M.ref(); o.has_cin = true;
      o.alpha = 1.0; o.beta = -kTay1; o.gamma = kTay0 + kTay1;
    } else {  // X' = X Q
      o.A = r.X.ref(); o.B = r.Q.ref(); o.C = r.Xn;
    }
    return o;
  }
  if (stage == 0 && job == 0) {  // T2 = ((M/s)^2 - 10 M/s + 25 I) / 16
    o.A = r.M.ref(); o.B = r.M.ref(); o.C = r.T2; o.Cin = r.M.ref(); o.has_cin = true;
    o.alpha = is * is / 16.0; o.beta = -10.0 * is / 16.0; o.gamma = 25.0 / 16.0;
  } else if (stage == 0) {  // X' = s^(-1/4) (5 X - X M/s) / 4
    const double q = pow(s, -0.25);
    o.A = r.X.ref(); o.B = xm ? r.Mx.ref() : r.M.ref(); o.C = r.Xn; o.Cin = r.X.ref(); o.has_cin = true;
    o.alpha = -0.25 * q * is; o.beta = 1.25 * q;
  } else if (stage == 1) {  // T4 = T2 T2
    o.A = r.T2.ref(); o.B = r.T2.ref(); o.C = r.T4;
  } else {  // M' = T4 M / s, written over T2
    o.A = r.T4.ref(); o.B = r.M.ref(); o.C = r.T2;
    o.alpha = is;
  }
  return o;
}

template <int VEC>
__global__ __launch_bounds__(256, 2) void newton_x3_kernel(const NewtonLaunch L, int kind) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[X3Tile::LDS_HALVES];
  const StageJob s = stage_job(L, kind);
  if (!s.active) return;
  const RolesS r = roless(s.region, s.d, L.t);
  const SplitOps o = split_ops(r, L.stage, s.job, s.s, kind == kStageX3B64, s.fin);
  const int m0 = s.ti * X3Tile::BM, n0 = s.tj * X3Tile::BN;
  v16f acc[2][2];
  x3_nt_tile_auto<VEC>(o.A, s.d, o.B, s.d, s.d, s.d, s.d, m0, n0, reinterpret_cast<unsigned char*>(smem), acc);
  const int d = s.d;
  const bool whole = VEC == 8 && s.ti <= s.tj && m0 + X3Tile::BM <= d && n0 + X3Tile::BN <= d;
  static_assert(4 * kSlabFloats * 4 <= (int)sizeof(smem), "four slabs fit in the operand stages");
  // Whole tile on or above the diagonal: the upper elements and their mirror
  // with wide stores through per-wave LDS slabs (the main loop ended with a
  // block barrier, so the operand stages are free); else element stores.
  auto store = [&](const SplitBuf& C, double al, double be, double ga) __attribute__((always_inline)) {
    if (whole) {
      wide_store_tile<2, 2, double>(acc, reinterpret_cast<float*>(smem), m0, n0, C.hi, C.lo, d, C.hi, C.lo, d,
                                    o.has_cin ? o.Cin.hi : nullptr, o.has_cin ? o.Cin.lo : nullptr, al, be, ga,
                                    s.ti == s.tj);
      return;
    }
    f32_for_each(acc, [&](int rr, int cc, float v) {
      const int gr = m0 + rr, gc = n0 + cc;
      if (gr < d && gc < d && gr <= gc) {
        const int64_t e = (int64_t)gr * d + gc;
        double val = al * (double)v;
        if (o.has_cin) val += be * (double)join_f32(o.Cin.hi[e], o.Cin.lo[e]);
        if (gr == gc) val += ga;
        split_put(C, e, (float)val);
        if (gr != gc) split_put(C, (int64_t)gc * d + gr, (float)val);
      }
    });
  };
  if (!o.has_c2) {
    store(o.C, o.alpha, o.beta, o.gamma);
  } else {  // two outputs of one product (degree-4 finish)
    store(o.C, o.alpha, o.beta, o.gamma);
    store(o.C2, o.alpha2, o.beta2, o.gamma2);
  }
}

// The same stages on 256 x 256 tiles with the single-accumulator split core
// (x3w_nt_tile).  Its B operands are M, the split copy Mx of a float64 M, or
// T2, whose spectra lie in [0, 1] and [1/4, 25/16] (u/s <= 3 in these steps,
// the float64 steps' M <= 1), or in a finishing step R (in [0.15, 0.17]) or
// q(M) (in [1, 1.03]), so every |B| < 2 and the 2^11 scaling of B's hi half
// stays far inside fp16's range.  The host picks this kernel for
// classes with d a multiple of 32 (whole 32-deep chunks) and d >= kWideMinD.
__global__ __launch_bounds__(X3W::THREADS, 1) void newton_x3w_kernel(const NewtonLaunch L, int kind) {
  constexpr int kSmem = X3W::LDS_BYTES > 8 * kSlabFloats * 4 ? X3W::LDS_BYTES : 8 * kSlabFloats * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  const StageJob s = stage_job(L, kind);
  if (!s.active) return;
  const RolesS r = roless(s.region, s.d, L.t);
  const SplitOps o = split_ops(r, L.stage, s.job, s.s, kind == kStageX3B64, s.fin);
  const int m0 = s.ti * X3W::BM, n0 = s.tj * X3W::BN;
  const int d = s.d;
  v16f acc[X3W::RB][X3W::CB];
  x3w_nt_tile(o.A, d, o.B, d, d, d, d, m0, n0, smem, acc);
  const bool whole = s.ti <= s.tj && m0 + X3W::BM <= d && n0 + X3W::BN <= d;
  // whole tile on or above the diagonal: wide stores through per-wave slabs;
  // else element stores
  auto store = [&](const SplitBuf& C, double al, double be, double ga) __attribute__((always_inline)) {
    if (whole) {
      wide_store_tile<X3W::RB, X3W::WN, double, X3W::CB>(
          acc, reinterpret_cast<float*>(smem), m0, n0, C.hi, C.lo, d, C.hi, C.lo, d,
          o.has_cin ? o.Cin.hi : nullptr, o.has_cin ? o.Cin.lo : nullptr, al, be, ga, s.ti == s.tj);
      return;
    }
    x3w_for_each(acc, [&](int rr, int cc, float v) {
      const int gr = m0 + rr, gc = n0 + cc;
      if (gr < d && gc < d && gr <= gc) {
        const int64_t e = (int64_t)gr * d + gc;
        double val = al * (double)v;
        if (o.has_cin) val += be * (double)join_f32(o.Cin.hi[e], o.Cin.lo[e]);
        if (gr == gc) val += ga;
        split_put(C, e, (float)val);
        if (gr != gc) split_put(C, (int64_t)gc * d + gr, (float)val);
      }
    });
  };
  if (!o.has_c2) {
    store(o.C, o.alpha, o.beta, o.gamma);
  } else {  // two outputs of one product (degree-4 finish)
    store(o.C, o.alpha, o.beta, o.gamma);
    store(o.C2, o.alpha2, o.beta2, o.gamma2);
  }
}

// 16 values -> their digits at byte offset `off` of each plane, one 16-byte
// store per plane.
__device__ __forceinline__ void oz_store16(const double (&w)[16], int e, const OzPlanes& P, int64_t off) {
  uint32_t pk[kOzSlices][4];
#pragma unroll
  for (int p = 0; p < kOzSlices; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) pk[p][q] = 0u;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int8_t dg[kOzSlices];
    oz_digits(w[k], e, dg);
#pragma unroll
    for (int p = 0; p < kOzSlices; ++p) pk[p][k >> 2] |= (uint32_t)(uint8_t)dg[p] << (8 * (k & 3));
  }
#pragma unroll
  for (int p = 0; p < kOzSlices; ++p)
    *reinterpret_cast<v4i*>(P.p[p] + off) = v4i{(int)pk[p][0], (int)pk[p][1], (int)pk[p][2], (int)pk[p][3]};
}

// ------------------------------------------------ int8 digit-plane steps
// Float64 steps of the split-storage path: the products of M, T2 and T4 run
// on int8 digit planes (gemm_i8.hpp).  M gets one exponent per row, cut from
// the float64 M at the start of each step by a pass of its own: its entries
// can sit far below its spectral bound (a log-uniform spectrum puts the
// diagonal near the mean eigenvalue), and a fixed exponent there loses
// enough digits to show in the root.  T2 and T4 take the fixed exponents 1
// and 2 (spectra in [0, 25/16] and [0, 625/256]: T = (5 I - M/s)/4 with the
// spectrum of M/s in [0, 4.8], so their diagonals, and with them their
// largest entries, sit near the top of those ranges), and their planes come
// straight from the product epilogues.  Stage 2 writes the float64 M' and its
// split copy, as the float64 kernel does.
// Plane positions (oz_layout): M's planes are persistent planes 0..5, T4's
// 6..11; T2's at iteration t are in the float64 slot M' of iteration t takes.
struct OzRegion {
  OzPlanes M, T2, T4;
  int32_t* eM;  // M's row exponents
  int64_t dp;
};
__host__ __device__ __forceinline__ OzRegion oz_region(char* region, int d, int t) {
  const OzLayout ly = oz_layout(d);
  const int64_t d2 = (int64_t)d * d;
  char* extra = region + oz_f64_bytes(d);
  char* over = extra + oz_align256(4 * oz_pad(d));
  auto persistent = [&](int i) -> int8_t* {
    if (i < ly.n_slot4) return reinterpret_cast<int8_t*>(region + 32 * d2 + i * ly.plane);
    if (i < ly.n_slot4 + ly.n_half3)
      return reinterpret_cast<int8_t*>(region + 12 * d2 + (i - ly.n_slot4) * ly.plane);
    return reinterpret_cast<int8_t*>(over + (i - ly.n_slot4 - ly.n_half3) * ly.plane);
  };
  OzRegion z;
#pragma unroll
  for (int p = 0; p < kOzSlices; ++p) {
    z.M.p[p] = persistent(p);
    z.T4.p[p] = persistent(kOzSlices + p);
    z.T2.p[p] = ly.t2_in_slot
                    ? reinterpret_cast<int8_t*>(reinterpret_cast<char*>(roles64(region, d, t).T2) + p * ly.plane)
                    : reinterpret_cast<int8_t*>(over + (2 * kOzSlices - ly.n_slot4 - ly.n_half3 + p) * ly.plane);
  }
  z.eM = reinterpret_cast<int32_t*>(extra);
  z.dp = oz_pad(d);
  return z;
}
constexpr int kOzExpT2 = 1, kOzExpT4 = 2;

// Digit planes of M (iteration t) with per-row exponents: a wave per padded
// row, kOzSliceRows (16) rows per workgroup (a long schedule launches this
// pass for every step it might need, and most workgroups exit at once); each
// lane takes 16-element segments 1024 elements apart, reads them for the
// row's largest magnitude and again (from cache) for the digits.  Rows and
// columns past d get zero digits (and rows exponent 0).  Runs for the
// matrices whose step t is a float64 step with products (t < j, t < K - 1).
__global__ __launch_bounds__(256) void newton_slice_kernel(const NewtonLaunch L) {
  const int64_t b = blockIdx.x;
  const NewtonClass& C = L.cls[find_class(L, b)];
  const int local = (int)(b - C.block_begin);
  if (local >= C.nblocks) return;
  const int mat = local / C.blocks_per_matrix;
  const int row0 = (local % C.blocks_per_matrix) * kOzSliceRows;
  const RootState& st = L.state[C.slot_begin + mat];
  const int t = L.t;
  if (!(t < st.j && t < st.K - 1)) return;
  const int d = C.d;
  char* region = C.region + (int64_t)mat * C.matrix_bytes;
  const OzRegion z = oz_region(region, d, t);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool vec = (d & 1) == 0;  // 16-byte loads (rows 16-byte aligned)
  for (int row = row0 + wave; row < row0 + kOzSliceRows; row += 4) {
    const double* M = roles64(region, d, t).M + (int64_t)row * d;
    const bool real = row < d;
    auto load16 = [&](int c0, double (&w)[16]) __attribute__((always_inline)) {
      if (real && vec && c0 + 16 <= d) {
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          const v2d x = *reinterpret_cast<const v2d*>(M + c0 + k);
          w[k] = x[0];
          w[k + 1] = x[1];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = real && c0 + k < d ? M[c0 + k] : 0.0;
      }
    };
    double mx = 0.0;
    for (int c0 = lane * 16; c0 < z.dp; c0 += 64 * 16) {
      double w[16];
      load16(c0, w);
#pragma unroll
      for (int k = 0; k < 16; ++k) mx = fmax(mx, fabs(w[k]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    int e = 0;
    if (mx > 0.0) frexp(mx, &e);  // mx < 2^e
    if (lane == 0) z.eM[row] = e;
    for (int c0 = lane * 16; c0 < z.dp; c0 += 64 * 16) {
      double w[16];
      load16(c0, w);
      oz_store16(w, e, z.M, (int64_t)row * z.dp + c0);
    }
  }
}

// One 128 x 128 upper tile of a float64 step's product on the digit planes:
//   stage 0: T2 = ((M/s)^2 - 10 M/s + 25 I) / 16   -> T2 planes
//   stage 1: T4 = T2 T2                            -> T4 planes
//   stage 2: M' = T4 M / s                         -> float64 M' and its split copy
// The tile goes through LDS (in the operand stages the main loop has
// released) as float64 values: row pitch kOzOutLd doubles (16 banks apart),
// columns interleaved by 16-element segment with the segment index XORed
// with r / 16, so that a row's eight segments and a column's eight 16-row
// groups both read on distinct banks.  It leaves as rows: eight lanes write
// one row of the tile, or of its mirror, 16 elements each, so every store
// instruction fills whole 128-byte lines.  Stages 0 and 1 cut each value
// into its digits once: a lane takes two row segments, stores their digits
// as the tile's rows and keeps them in six 128 x 128 byte planes (byte
// (r, c) in row r, segment (c / 16) XOR (r / 16 mod 8)), from which the
// mirror's rows are gathered a byte at a time.  Outside the d x d matrix the
// planes get zeros.
constexpr int kOzOutLd = kOzTile + 8;
constexpr int kOzPlaneBytes = kOzTile * kOzTile;
__device__ __forceinline__ int oz_tpos(int r, int c) {
  return r * kOzOutLd + ((c & 15) << 3) + ((c >> 4) ^ ((r >> 4) & 7));
}
__device__ __forceinline__ int oz_bpos(int r, int c) {
  return r * kOzTile + ((((c >> 4) ^ (r >> 4)) & 7) << 4) + (c & 15);
}
__global__ __launch_bounds__(OzCfg::THREADS, 1) void newton_i8_kernel(const NewtonLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[OzCfg::LDS_BYTES];
  static_assert(kOzTile * kOzOutLd * 8 + 2 * kOzTile * 4 <= OzCfg::LDS_BYTES,
                "the float64 tile and its exponents fit in the operand stages");
  static_assert(kOzSlices * kOzPlaneBytes <= OzCfg::LDS_BYTES, "the byte planes fit in the operand stages");
  static_assert(kOzTile == 128, "eight 16-element segments per row, eight 16-row groups per column");
  const StageJob s = stage_job(L, kStageI8);
  if (!s.active) return;
  const int d = s.d;
  const int stage = L.stage;
  const OzRegion z = oz_region(s.region, d, L.t);
  const int64_t dp = z.dp;
  OzPlanes A, B;  // by value: a reference picked at run time would put z in scratch memory
#pragma unroll
  for (int p = 0; p < kOzSlices; ++p) {
    A.p[p] = stage == 0 ? z.M.p[p] : stage == 1 ? z.T2.p[p] : z.T4.p[p];
    B.p[p] = stage == 1 ? z.T2.p[p] : z.M.p[p];
  }
  const int m0 = s.ti * kOzTile, n0 = s.tj * kOzTile;
  v16i acc[kOzSlices][2];
  oz_nt_tile(A, B, dp, (int)dp, m0, n0, smem, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const Roles64 r64 = roles64(s.region, d, L.t);
  const double is = 1.0 / s.s;
  const bool diag = s.ti == s.tj;
  // the unscaled sums into LDS, the operands' exponents of the tile's rows
  // (E[0..127]) and columns (E[128..255]) after them
  double* T = reinterpret_cast<double*>(smem);
  int* E = reinterpret_cast<int*>(smem + kOzTile * kOzOutLd * 8);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int li = wm * 32 + f32_row(lane, v);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) T[oz_tpos(li, wn * 64 + cb * 32 + (lane & 31))] = oz_value(acc, cb, v, 12);
  }
  if (threadIdx.x < 2 * kOzTile) {
    const int i = threadIdx.x & (kOzTile - 1);
    E[threadIdx.x] = threadIdx.x < kOzTile ? (stage == 0 ? z.eM[m0 + i] : stage == 1 ? kOzExpT2 : kOzExpT4)
                                           : (stage == 1 ? kOzExpT2 : z.eM[n0 + i]);
  }
  __syncthreads();
  // product element (m0 + a, n0 + b), as float64
  auto prod = [&](int a, int b) __attribute__((always_inline)) {
    return ldexp(T[oz_tpos(a, b)], E[a] + E[kOzTile + b] - 12);
  };
  if (stage < 2) {
    // each lane takes two 16-element row segments of the tile: their values,
    // then (the float64 tile released) their digits, stored as the tile's
    // rows and kept in the byte planes for the mirror
    constexpr int kSeg = kOzTile * (kOzTile / 16) / OzCfg::THREADS;
    double w[kSeg][16];
#pragma unroll
    for (int it = 0; it < kSeg; ++it) {
      const int q = threadIdx.x + it * OzCfg::THREADS;
      const int lr = q >> 3, c0 = (q & 7) * 16;
      const int gi = m0 + lr;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int gj = n0 + c0 + k;
        const double x = prod(lr, c0 + k);
        double val = 0.0;
        if (gi < d && gj < d)
          val = stage == 0 ? x * (is * is / 16.0) - (10.0 * is / 16.0) * r64.M[(int64_t)gi * d + gj] +
                                 (gi == gj ? 25.0 / 16.0 : 0.0)
                           : x;
        w[it][k] = val;
      }
    }
    __syncthreads();
    unsigned char* Dg = smem;
    OzPlanes out;
#pragma unroll
    for (int p = 0; p < kOzSlices; ++p) out.p[p] = stage == 0 ? z.T2.p[p] : z.T4.p[p];
    const int eo = stage == 0 ? kOzExpT2 : kOzExpT4;
#pragma unroll
    for (int it = 0; it < kSeg; ++it) {
      const int q = threadIdx.x + it * OzCfg::THREADS;
      const int lr = q >> 3, c0 = (q & 7) * 16;
      uint32_t pk[kOzSlices][4];
#pragma unroll
      for (int p = 0; p < kOzSlices; ++p)
#pragma unroll
        for (int u = 0; u < 4; ++u) pk[p][u] = 0u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        int8_t dg[kOzSlices];
        oz_digits(w[it][k], eo, dg);
#pragma unroll
        for (int p = 0; p < kOzSlices; ++p) pk[p][k >> 2] |= (uint32_t)(uint8_t)dg[p] << (8 * (k & 3));
      }
      const int64_t off = (int64_t)(m0 + lr) * dp + n0 + c0;
#pragma unroll
      for (int p = 0; p < kOzSlices; ++p) {
        const v4i x = v4i{(int)pk[p][0], (int)pk[p][1], (int)pk[p][2], (int)pk[p][3]};
        *reinterpret_cast<v4i*>(Dg + p * kOzPlaneBytes + oz_bpos(lr, c0)) = x;
        if (!diag) *reinterpret_cast<v4i*>(out.p[p] + off) = x;
      }
    }
    __syncthreads();
    // on the diagonal: the tile's region (upper bytes, mirrored below); else
    // the mirror region (n0.., m0..)
    const int R0 = diag ? m0 : n0, C0 = diag ? n0 : m0;
    for (int q = threadIdx.x; q < kOzTile * (kOzTile / 16); q += OzCfg::THREADS) {
      const int lr = q >> 3, c0 = (q & 7) * 16;
      const int64_t off = (int64_t)(R0 + lr) * dp + C0 + c0;
#pragma unroll
      for (int p = 0; p < kOzSlices; ++p) {
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int lc = c0 + k;
          const bool mir = !diag || lr > lc;
          const uint32_t bt = Dg[p * kOzPlaneBytes + (mir ? oz_bpos(lc, lr) : oz_bpos(lr, lc))];
          wv[k >> 2] |= bt << (8 * (k & 3));
        }
        *reinterpret_cast<v4i*>(out.p[p] + off) = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
      }
    }
    return;
  }

  const SplitBuf mx = roless(s.region, d, L.t).Mx;
  for (int pass = 0; pass < (diag ? 1 : 2); ++pass) {
    const int R0 = pass == 0 ? m0 : n0, C0 = pass == 0 ? n0 : m0;
    for (int q = threadIdx.x; q < kOzTile * (kOzTile / 16); q += OzCfg::THREADS) {
      const int lr = q >> 3, c0 = (q & 7) * 16;
      const int gi = R0 + lr, gj0 = C0 + c0;
      if (gi >= d) continue;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int lc = c0 + k, gj = gj0 + k;
        if (gj < d) {
          const double w = ((pass == 1 || (diag && lr > lc)) ? prod(lc, lr) : prod(lr, lc)) * is;
          const int64_t e = (int64_t)gi * d + gj;
          r64.T2[e] = w;
          split_put(mx, e, (float)w);
        }
      }
    }
  }
}

// float64 M, X of iteration t -> float32 M, X of iteration t, for the
// matrices whose switch iteration is t.
__global__ __launch_bounds__(256) void newton_convert_kernel(const NewtonLaunch L) {
  const int64_t b = blockIdx.x;
  const NewtonClass& C = L.cls[find_class(L, b)];
  const int local = (int)(b - C.block_begin);
  if (local >= C.nblocks) return;
  const int mat = local / C.blocks_per_matrix;
  const int chunk = local % C.blocks_per_matrix;
  const RootState& st = L.state[C.slot_begin + mat];
  const int t = L.t;
  if (!(st.j == t && t < st.K)) return;
  char* region = C.region + (int64_t)mat * C.matrix_bytes;
  const Roles64 r64 = roles64(region, C.d, t);
  const Roles32 r32 = roles32(region, C.d, t);
  const int64_t n = (int64_t)C.d * C.d;
  const int64_t per = 256 * 8;
  const int64_t e0 = (int64_t)chunk * per;
  if (L.x_low) {
    const SplitBuf ms = roless(region, C.d, t).M;
    for (int64_t e = e0 + threadIdx.x; e < min(n, e0 + per); e += 256) split_put(ms, e, (float)r64.M[e]);
  } else {
    for (int64_t e = e0 + threadIdx.x; e < min(n, e0 + per); e += 256) {
      r32.M[e] = (float)r64.M[e];
      r32.X[e] = (float)r64.X[e];
    }
  }
}

// ------------------------------------------------------------ finalize
// X_out = c^(-1/4) X_K (float32), plus per-row-block partial sums of
// |M_{K-1} - I|^2 for the residual.  Flagged matrices get their special
// outputs: NaN (non-finite input / no usable bound), eps^(-1/4) I (zero trace).
__global__ __launch_bounds__(256) void root_finalize_kernel(const RootBatch B) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_job(B, b)];
  const int blk = (int)(b - J.block_begin);
  const RootState& st = B.state[J.slot];
  const int d = J.d;
  const int r0 = blk * kFinalRows, r1 = min(d, r0 + kFinalRows);
  double res = 0.0;
  if (st.K == 0) {
    const bool zero_trace = (st.flags & MR_INFO_ZERO_TRACE) != 0;
    const float diag = zero_trace ? (float)pow(B.eps, -0.25) : __builtin_nanf("");
    const float off = zero_trace ? 0.f : __builtin_nanf("");
    for (int r = r0; r < r1; ++r)
      for (int c = threadIdx.x; c < d; c += 256) J.X[(int64_t)r * J.ldx + c] = (r == c) ? diag : off;
  } else {
    const int K = st.K, j = st.j;
    const double sc = st.out_scale;
    const bool x64 = K <= j;
    const bool m64 = (K - 1) < j;
    const Roles64 rx64 = roles64(J.region, d, K), rm64 = roles64(J.region, d, K - 1);
    const Roles32 rx32 = roles32(J.region, d, K), rm32 = roles32(J.region, d, K - 1);
    const RolesS rxs = roless(J.region, d, K), rms = roless(J.region, d, K - 1);
    const double xsc = B.x_low ? sc / (double)x_store_scale(st) : sc;
    for (int r = r0; r < r1; ++r) {
      for (int c = threadIdx.x; c < d; c += 256) {
        const int64_t e = (int64_t)r * d + c;
        double x, m;
        if (B.x_low) {
          x = (double)join_f32(rxs.X.hi[e], rxs.X.lo[e]);
          m = m64 ? rm64.M[e] : (double)join_f32(rms.M.hi[e], rms.M.lo[e]);
        } else {
          x = x64 ? rx64.X[e] : (double)rx32.X[e];
          m = m64 ? rm64.M[e] : (double)rm32.M[e];
        }
        J.X[(int64_t)r * J.ldx + c] = (float)(xsc * x);
        m -= (r == c ? 1.0 : 0.0);
        res += m * m;
      }
    }
  }
  res = block_sum_256(res, red);
  if (threadIdx.x == 0) B.partial[(int64_t)J.slot * B.partial_stride + blk] = res;
}

// One wave per slot: residual of Newton matrices, convergence flag, info.
__global__ __launch_bounds__(64) void root_info_kernel(RootState* state, const double* partial, int64_t stride,
                                                       mr_root_info* info) {
  __shared__ double red[64];
  RootState& st = state[blockIdx.x];
  const bool newton = st.method == MR_NEWTON;
  double res = 0.0;
  if (newton) {
    const int nb = (st.d + kFinalRows - 1) / kFinalRows;
    const double* p = partial + (int64_t)blockIdx.x * stride;
    for (int i = threadIdx.x; i < nb; i += 64) res += p[i];
  }
  res = block_sum_64(res, red);
  if (threadIdx.x != 0) return;
  if (newton && st.K > 0) {
    const double r = sqrt(res);
    st.residual = (float)r;
    // rms deviation the last X update may start from: that of the plain step,
    // or 1.5 times the spectrum radius a Taylor finish accepts
    const double rms = st.fin == 2 ? 1.5 * kFinishQuad : st.fin == 4 ? 1.5 * kFinishQuartic : 2e-3;
    if (!(r <= rms * sqrt((double)st.d))) st.flags |= MR_INFO_NOT_CONVERGED;
  }
  if (info) {
    mr_root_info o;
    o.scale = st.s;
    o.bound = newton ? st.c : 0.0;
    o.iters = newton ? st.K : st.sweeps;
    o.fp64_iters = newton ? min(st.j, st.K) : 0;
    o.residual = st.residual;
    o.flags = st.flags;
    o.final_degree = newton ? st.fin : 0;
    o.reserved = 0;
    info[st.problem] = o;
  }
}

// ------------------------------------------------------------ launchers
hipError_t launch_root_stats(const RootBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (b.a_f64)
    hipLaunchKernelGGL(root_stats_kernel<double>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(root_stats_kernel<float>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_root_bound(RootState* state, double* partial, int64_t partial_stride, double* sched,
                             int32_t slot_begin, int32_t nslots, int32_t normalize, double eps, int32_t k_cap,
                             double floor_cap, int32_t all_f64, int32_t finish, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  hipLaunchKernelGGL(root_bound_kernel, dim3(nslots), dim3(64), 0, s, state, partial, partial_stride, sched,
                     slot_begin, normalize, eps, k_cap, floor_cap, all_f64, finish);
  return hipGetLastError();
}

hipError_t launch_root_moment_convert(const RootBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (b.a_f64)
    hipLaunchKernelGGL(root_moment_convert_kernel<double>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(root_moment_convert_kernel<float>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_root_moment(const RootBatch& b, int pass, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (pass == 0)
    hipLaunchKernelGGL(root_moment_kernel<0>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(root_moment_kernel<1>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_root_tighten(RootState* state, const double* partial, int64_t partial_stride, double* sched,
                               int32_t slot_begin, int32_t nslots, double eps, int32_t k_cap, double floor_cap,
                               int32_t all_f64, int32_t finish, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  hipLaunchKernelGGL(root_tighten_kernel, dim3(nslots), dim3(64), 0, s, state, partial, partial_stride, sched,
                     slot_begin, eps, k_cap, floor_cap, all_f64, finish);
  return hipGetLastError();
}

hipError_t launch_root_init(const RootBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (b.a_f64)
    hipLaunchKernelGGL(root_init_kernel<double>, dim3(b.total_blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(root_init_kernel<float>, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_newton_stage(const NewtonLaunch& L, int kind, int vec, hipStream_t s) {
  if (L.total_blocks <= 0) return hipSuccess;
  if (kind == kStageX3 || kind == kStageX3B64) {
    if (L.wide)
      hipLaunchKernelGGL(newton_x3w_kernel, dim3(L.total_blocks), dim3(X3W::THREADS), 0, s, L, kind);
    else if (vec >= 8)
      hipLaunchKernelGGL(newton_x3_kernel<8>, dim3(L.total_blocks), dim3(256), 0, s, L, kind);
    else
      hipLaunchKernelGGL(newton_x3_kernel<1>, dim3(L.total_blocks), dim3(256), 0, s, L, kind);
    return hipGetLastError();
  }
  if (kind == kStageI8) {
    hipLaunchKernelGGL(newton_i8_kernel, dim3(L.total_blocks), dim3(OzCfg::THREADS), 0, s, L);
    return hipGetLastError();
  }
  if (kind == kStageF64) {
    if (vec > 1)
      hipLaunchKernelGGL(newton_f64_kernel<2>, dim3(L.total_blocks), dim3(256), 0, s, L);
    else
      hipLaunchKernelGGL(newton_f64_kernel<1>, dim3(L.total_blocks), dim3(256), 0, s, L);
  } else {
    if (vec == 4)
      hipLaunchKernelGGL(newton_f32_kernel<4>, dim3(L.total_blocks), dim3(256), 0, s, L);
    else
      hipLaunchKernelGGL(newton_f32_kernel<1>, dim3(L.total_blocks), dim3(256), 0, s, L);
  }
  return hipGetLastError();
}

hipError_t launch_newton_slice(const NewtonLaunch& L, hipStream_t s) {
  if (L.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(newton_slice_kernel, dim3(L.total_blocks), dim3(256), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_newton_convert(const NewtonLaunch& L, hipStream_t s) {
  if (L.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(newton_convert_kernel, dim3(L.total_blocks), dim3(256), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_root_finalize(const RootBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(root_finalize_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_root_info(RootState* state, const double* partial, int64_t partial_stride, int32_t count,
                            mr_root_info* info, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(root_info_kernel, dim3(count), dim3(64), 0, s, state, partial, partial_stride, info);
  return hipGetLastError();
}

}  // namespace mr
