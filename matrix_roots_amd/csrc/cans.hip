// W = S^(-1/2), S = (A + A^T)/2 / s + eps I, by the scaled CANS coupled
// Newton-Schulz iteration (tilderesearch, "Online KL Shampoo", sections
// 2.2-2.4 and appendix D; the recurrence, coefficients and scales are in
// cans.hpp).
//
// Per matrix: statistics (root_stats_kernel) -> bound L = 1.01 WS(S) and the
// output scale -> init (Y0 and Z1 = a0 I + b0 Y0, elementwise) -> 19 GEMM
// launches -> finalize (W = Z_10 / sqrt(L), residual ||P_9 - I||_F) -> info.
//
// Storage: Y, Z and P live in split form, hi = fp16(x) and lo =
// fp16((x - hi) 2^11), each times its step's power-of-two scale.  hi is
// exactly the fp16 cast the page feeds to its GEMMs; hi + 2^-11 lo keeps
// float32-level accuracy for the a_k Y and a_k Z terms, which the page keeps
// in float32.  Precision 1 multiplies hi by hi (the page's fp16 products with
// float32 accumulation); precision 3 adds the two cross terms with lo
// (float32-accurate products, as in the quarter root's float32 phase).
#include <math.h>

#include <type_traits>

#include "cans.hpp"
#include "epilogue.hpp"
#include "gemm_core.hpp"
#include "gemm_h16.hpp"

namespace mr {

namespace {

struct Split {
  _Float16* hi;
  _Float16* lo;
  __device__ __forceinline__ SplitRef ref() const { return SplitRef{hi, lo}; }
};

__device__ __forceinline__ Split cans_buf(char* region, int d, int i) {
  const int64_t n = (int64_t)d * d;
  _Float16* h = reinterpret_cast<_Float16*>(region + (int64_t)i * 4 * n);
  return Split{h, h + n};
}
__device__ __forceinline__ int buf_y(int k) { return k & 1; }
__device__ __forceinline__ int buf_z(int k) { return 2 + (k & 1); }
constexpr int kBufP = 4, kBufPt = 5;

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

__device__ __forceinline__ int find_root_job(const RootBatch& B, int64_t b) {
  int jx = 0;
  while (jx + 1 < B.njobs && b >= B.job[jx + 1].block_begin) ++jx;
  return jx;
}

}  // namespace

// One wave per matrix: combine the statistics partials (trace, sum of
// squares, non-finite count per row block, in a fixed order) into s, the
// bound L = 1.01 WS(S) on lambda_max(S) and the output scale.  WS is the
// Wolkowicz-Styan bound (the page bounds the largest eigenvalue by the
// smaller of this and a second bound before its iteration).
__global__ __launch_bounds__(64) void cans_bound_kernel(RootState* state, const double* partial, int64_t stride,
                                                        int32_t nslots, int32_t normalize, double eps,
                                                        double z_out_scale) {
  __shared__ double red[64];
  const int slot = blockIdx.x;
  if (slot >= nslots) return;
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
  tr = block_sum(tr, red, 64);
  f2 = block_sum(f2, red, 64);
  nf = block_sum(nf, red, 64);
  if (threadIdx.x != 0) return;
  uint32_t flags = 0;
  double s = 1.0, L = 1.0;
  int K = 0;
  if (nf > 0.0 || !isfinite(tr) || !isfinite(f2)) {
    flags |= MR_INFO_NONFINITE;
  } else {
    if (normalize == MR_NORM_TRACE) s = tr;
    if (normalize == MR_NORM_TRACE && s == 0.0) {
      flags |= MR_INFO_ZERO_TRACE;
      if (!(eps > 0.0)) flags |= MR_INFO_NOT_PD;
    } else {
      const double dd = (double)d;
      const double trh = tr / s, f2h = f2 / (s * s);
      const double trS = trh + dd * eps;
      const double f2S = f2h + 2.0 * eps * trh + dd * eps * eps;
      const double m = trS / dd;
      const double ws = m + sqrt(fmax(f2S / dd - m * m, 0.0)) * sqrt(fmax(dd - 1.0, 0.0));
      L = kBoundSafety * ws;
      if (!(L > 0.0) || !isfinite(L)) {
        flags |= MR_INFO_NOT_PD;
        L = 1.0;
      } else {
        K = kCansSteps;
      }
    }
  }
  st.s = s;
  st.c = L;
  st.out_scale = 1.0 / (z_out_scale * sqrt(L));
  st.K = K;
  st.j = 0;
  st.flags = flags;
  st.method = kCansMethod;
  st.residual = 0.f;
}

// Y0 = sy0 S / L into Y(even) and Z1 = (za + zb y0) -- the scaled
// a0 I + b0 Y0 -- into Z(odd), 32 x 32 tiles of the symmetric part through
// LDS (load_sym_tile).
template <typename TA>
__global__ __launch_bounds__(256) void cans_init_kernel(const RootBatch B, double sy0, double za, double zb) {
  __shared__ double ta[32][33];
  __shared__ double tb[32][33];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_root_job(B, b)];
  const RootState& st = B.state[J.slot];
  if (st.K == 0) return;
  const int d = J.d;
  const int Tt = (d + 31) / 32;
  int bi, bj;
  upper_pair((int)(b - J.block_begin), Tt, bi, bj);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bool packed = B.a_packed != 0;
  load_sym_tile<TA>(J.A, J.lda, d, packed, bi, bj, ta, tb);
  const double inv_s = 1.0 / st.s, inv_L = 1.0 / st.c, eps = B.eps;
  const Split Y = cans_buf(J.region, d, buf_y(0));
  const Split Z = cans_buf(J.region, d, buf_z(1));
  auto put_yz = [&](int gi, int gj, double sym) __attribute__((always_inline)) {
    const double y0 = (sym * inv_s + (gi == gj ? eps : 0.0)) * inv_L;
    const int64_t i = (int64_t)gi * d + gj;
    put(Y, i, (float)(sy0 * y0));
    put(Z, i, (float)(zb * y0 + (gi == gj ? za : 0.0)));
  };
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = ty + 8 * e;
    // tile (bi, bj), then its mirror (bj, bi) from the same LDS tiles
    if (bi * 32 + r < d && bj * 32 + tx < d) put_yz(bi * 32 + r, bj * 32 + tx, sym_tile_value(packed, bi, bj, r, tx, ta, tb));
    if (bi != bj && bj * 32 + r < d && bi * 32 + tx < d)
      put_yz(bj * 32 + r, bi * 32 + tx, sym_tile_value(packed, bi, bj, tx, r, ta, tb));
  }
}

// Block shapes: split products use the 128 x 128 split core; fp16 products
// use kCansTile x kCansTile tiles (256: 8 waves of 128 x 64, each
// operand panel read half as often as with 128).
constexpr int kCansTile = 256;
constexpr int kCansBK = 32;
using CansSplitShape = H16Shape<128, 128, 2, 2>;
using CansF16Shape = H16Shape<kCansTile, kCansTile, 2, kCansTile / 64, kCansBK>;

// One launch stage of the iteration for every matrix of up to kMaxClasses
// size classes; workgroup -> (class, matrix, job, tile) through the per-class
// XCD remap.  PREC 1: fp16 products; PREC 3: split products.  FULL: the P
// stage (every tile, stored with its transpose); else the symmetric stages.
constexpr int kCansOccFull = 2;
constexpr int kCansOccSym = 2;
template <int VEC, int PREC, bool FULL, class S>
__global__ __launch_bounds__(S::THREADS, S::THREADS >= 512 ? 1
                                         : PREC == 3      ? 2
                                         : FULL           ? kCansOccFull
                                                          : kCansOccSym) void cans_gemm_kernel(const CansLaunch L) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[PREC == 3 ? 2 * X3Tile::LDS_HALVES : h16_kernel_lds_bytes<S>(4 * kSlabFloats)];
  const int64_t b = blockIdx.x;
  int ci = 0;
  while (ci + 1 < L.ncls && b >= L.cls[ci + 1].block_begin) ++ci;
  const CansClass& C = L.cls[ci];
  const int local = (int)xcd_remap(b - C.block_begin, round8(C.nblocks));
  if (local >= C.nblocks) return;
  const int mat = local / C.blocks_per_matrix;
  const int rem = local % C.blocks_per_matrix;
  if (L.state[C.slot_begin + mat].K == 0) return;
  const int d = C.d;
  char* region = C.region + (int64_t)mat * C.matrix_bytes;
  const int k = L.k;
  constexpr bool full = FULL;
  int job = 0, ti, tj;
  if (full) {
    full_tile_grouped(rem, C.T, C.T, ti, tj);
  } else {
    job = L.stage == kCansYZ ? rem / C.U : (L.stage == kCansZ ? 1 : 0);
    upper_tile_grouped(rem % C.U, C.T, ti, tj);
  }
  // operands (C = A B^T), output, and the a_k term's input
  Split A, Bm, Out, Cin;
  if (L.stage == kCansY1) {
    A = Bm = Cin = cans_buf(region, d, buf_y(0));
    Out = cans_buf(region, d, buf_y(1));
  } else if (full) {
    A = cans_buf(region, d, buf_z(k));
    Bm = cans_buf(region, d, buf_y(k));
    Out = cans_buf(region, d, kBufP);
  } else if (job == 0) {  // Y Z Y = Y P = Y (P^T)^T
    A = Cin = cans_buf(region, d, buf_y(k));
    Bm = cans_buf(region, d, kBufPt);
    Out = cans_buf(region, d, buf_y(k + 1));
  } else {  // Z Y Z = Z P^T
    A = Cin = cans_buf(region, d, buf_z(k));
    Bm = cans_buf(region, d, kBufP);
    Out = cans_buf(region, d, buf_z(k + 1));
  }
  // Epilogue arithmetic: float64 for split products (float32-accurate
  // results), float32 for fp16 products (its rounding, even under the first
  // step's 18-fold cancellation, stays far below the fp16 product noise).
  using E = typename std::conditional<PREC == 3, double, float>::type;
  const E alpha = (E)L.alpha[job], beta = (E)L.beta[job];
  const int m0 = ti * S::BM, n0 = tj * S::BN;
  v16f acc[S::RB][S::CB];
  if constexpr (PREC == 3)
    x3_nt_tile_auto<VEC>(A.ref(), d, Bm.ref(), d, d, d, d, m0, n0, smem, acc);
  else
    h16_nt_tile_auto<S, VEC>(A.hi, d, Bm.hi, d, d, d, d, m0, n0, smem, acc);

  const bool whole = m0 + S::BM <= d && n0 + S::BN <= d;
  if (VEC == 8 && whole && (full || ti <= tj)) {
    // whole tile (P, or on or above the diagonal): wide stores of the tile
    // and of its transpose (P^T, or the mirror) through per-wave LDS slabs
    static_assert(S::CB == 2, "slab epilogue takes two 32-column blocks per wave");
    static_assert((S::THREADS / 64) * kSlabFloats * 4 <= (int)sizeof(smem), "one slab per wave fits in the LDS");
    const Split T = full ? cans_buf(region, d, kBufPt) : Out;
    // fp16 products read P and P^T as operands only (hi halves): P's lo half
    // is kept for the last step's residual, P^T's never
    const bool p_lo = PREC == 3 || k == kCansSteps - 1;
    _Float16* out_lo = full && !p_lo ? nullptr : Out.lo;
    _Float16* t_lo = full && PREC != 3 ? nullptr : T.lo;
    wide_store_tile<S::RB, S::WN, E>(acc, reinterpret_cast<float*>(smem), m0, n0, Out.hi, out_lo, d, T.hi, t_lo, d,
                                     full ? nullptr : Cin.hi, full ? nullptr : Cin.lo, alpha, beta, E(0),
                                     !full && ti == tj);
    return;
  }
  const Split Pt = cans_buf(region, d, kBufPt);
  h16g_for_each<S>(acc, [&](int rr, int cc, float a) {
    const int gr = m0 + rr, gc = n0 + cc;
    if (gr >= d || gc >= d) return;
    if (full) {
      const float v = (float)(alpha * (E)a);
      put(Out, (int64_t)gr * d + gc, v);
      put(Pt, (int64_t)gc * d + gr, v);
    } else if (gr <= gc) {
      const int64_t i = (int64_t)gr * d + gc;
      const float v = (float)(alpha * (E)a + beta * (E)get(Cin, i));
      put(Out, i, v);
      if (gr != gc) put(Out, (int64_t)gc * d + gr, v);
    }
  });
}

// W = out_scale * Z_10 (float32), plus per-row-block partial sums of
// |P_9 - I|^2 for the residual.  Flagged matrices: eps^(-1/2) I for a zero
// trace with eps > 0, NaN otherwise.
__global__ __launch_bounds__(256) void cans_finalize_kernel(const RootBatch B, double inv_sp9) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const RootJob& J = B.job[find_root_job(B, b)];
  const RootState& st = B.state[J.slot];
  const int d = J.d;
  const int blk = (int)(b - J.block_begin);
  const int r0 = blk * kFinalRows, r1 = min(d, r0 + kFinalRows);
  double res = 0.0;
  if (st.K == 0) {
    const bool zt = st.flags == MR_INFO_ZERO_TRACE;
    const float diag = zt ? (float)(1.0 / sqrt(B.eps)) : __builtin_nanf("");
    const float off = zt ? 0.f : __builtin_nanf("");
    for (int r = r0; r < r1; ++r)
      for (int c = threadIdx.x; c < d; c += 256) J.X[(int64_t)r * J.ldx + c] = r == c ? diag : off;
  } else {
    const Split Z = cans_buf(J.region, d, buf_z(kCansSteps));
    const Split P = cans_buf(J.region, d, kBufP);
    const double sc = st.out_scale;
    for (int r = r0; r < r1; ++r)
      for (int c = threadIdx.x; c < d; c += 256) {
        const int64_t i = (int64_t)r * d + c;
        J.X[(int64_t)r * J.ldx + c] = (float)(sc * (double)get(Z, i));
        const double e = (double)get(P, i) * inv_sp9 - (r == c ? 1.0 : 0.0);
        res += e * e;
      }
  }
  res = block_sum(res, red, 256);
  if (threadIdx.x == 0) B.partial[(int64_t)J.slot * B.partial_stride + blk] = res;
}

// One wave per slot: residual, convergence flag and the info record.
__global__ __launch_bounds__(64) void cans_info_kernel(RootState* state, const double* partial, int64_t stride,
                                                       int32_t count, mr_root_info* info, double rms_limit) {
  __shared__ double red[64];
  if ((int)blockIdx.x >= count) return;
  RootState& st = state[blockIdx.x];
  const int nb = (st.d + kFinalRows - 1) / kFinalRows;
  const double* p = partial + (int64_t)blockIdx.x * stride;
  double res = 0.0;
  for (int i = threadIdx.x; i < nb; i += 64) res += p[i];
  res = block_sum(res, red, 64);
  if (threadIdx.x != 0) return;
  if (st.K > 0) {
    const double r = sqrt(res);
    st.residual = (float)r;
    if (!(r <= rms_limit * sqrt((double)st.d))) st.flags |= MR_INFO_NOT_CONVERGED;
  }
  if (info) {
    mr_root_info o;
    o.scale = st.s;
    o.bound = st.c;
    o.iters = st.K;
    o.fp64_iters = 0;
    o.residual = st.residual;
    o.flags = st.flags;
    o.final_degree = 0;
    o.reserved = 0;
    info[st.problem] = o;
  }
}

// ------------------------------------------------------------ launchers
hipError_t launch_cans_bound(RootState* state, const double* partial, int64_t stride, int32_t nslots,
                             int32_t normalize, double eps, double z_out_scale, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  hipLaunchKernelGGL(cans_bound_kernel, dim3(nslots), dim3(64), 0, s, state, partial, stride, nslots, normalize,
                     eps, z_out_scale);
  return hipGetLastError();
}

hipError_t launch_cans_init(const RootBatch& b, double sy0, double za, double zb, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  if (b.a_f64)
    hipLaunchKernelGGL(cans_init_kernel<double>, dim3(b.total_blocks), dim3(256), 0, s, b, sy0, za, zb);
  else
    hipLaunchKernelGGL(cans_init_kernel<float>, dim3(b.total_blocks), dim3(256), 0, s, b, sy0, za, zb);
  return hipGetLastError();
}

int cans_tile(int prec) { return prec == 3 ? CansSplitShape::BM : CansF16Shape::BM; }

hipError_t launch_cans_gemm(const CansLaunch& L, int vec, int prec, hipStream_t s) {
  if (L.total_blocks <= 0) return hipSuccess;
  const dim3 g(L.total_blocks);
  const bool full = L.stage == kCansP;
#define MR_CANS_LAUNCH(V, P, SH)                                                                        \
  do {                                                                                                  \
    if (full)                                                                                           \
      hipLaunchKernelGGL((cans_gemm_kernel<V, P, true, SH>), g, dim3(SH::THREADS), 0, s, L);           \
    else                                                                                                \
      hipLaunchKernelGGL((cans_gemm_kernel<V, P, false, SH>), g, dim3(SH::THREADS), 0, s, L);          \
  } while (0)
  if (prec == 3) {
    if (vec == 8)
      MR_CANS_LAUNCH(8, 3, CansSplitShape);
    else
      MR_CANS_LAUNCH(1, 3, CansSplitShape);
  } else {
    if (vec == 8)
      MR_CANS_LAUNCH(8, 1, CansF16Shape);
    else
      MR_CANS_LAUNCH(1, 1, CansF16Shape);
  }
#undef MR_CANS_LAUNCH
  return hipGetLastError();
}

hipError_t launch_cans_finalize(const RootBatch& b, double inv_sp9, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(cans_finalize_kernel, dim3(b.total_blocks), dim3(256), 0, s, b, inv_sp9);
  return hipGetLastError();
}

hipError_t launch_cans_info(RootState* state, const double* partial, int64_t stride, int32_t count,
                            mr_root_info* info, double rms_limit, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(cans_info_kernel, dim3(count), dim3(64), 0, s, state, partial, stride, count, info,
                     rms_limit);
  return hipGetLastError();
}

}  // namespace mr
