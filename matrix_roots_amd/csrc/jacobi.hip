// Regularised inverse quarter root of small Grams (d <= 128) by an explicit
// eigendecomposition: one workgroup per matrix, the matrix held in LDS.
//
// The pages' step (marin.community, "Sharding EMA-Gram eigensolves", section
// "Background"): decompose the rescaled Gram into eigenvectors and
// eigenvalues, add a small regulariser to the eigenvalues, raise them to
// -1/4 and rebuild the matrix.  Here the decomposition is the cyclic Jacobi
// method in float64 with the round-robin ("chess tournament") ordering:
// each round rotates n/2 disjoint index pairs at once, so A <- J^T A J is a
// set of independent 2 x 2 block updates, and n - 1 rounds visit every pair
// once per sweep.  A rotation is skipped when |a_pq| <= 1e-15 |A|_F; the
// sweeps stop when a whole sweep rotates nothing.  Eigenvectors accumulate as
// rows of W = V^T.  Then, with f_k = (lambda_k + eps)^(-1/4),
// X = sum_k f_k v_k v_k^T is formed as W'^T W' with W' = diag(sqrt f) W,
// which is exactly symmetric.  Odd d is padded with a zero row and column
// that never rotates.
//
// Layout: a launch covers one size class (padded size NMAX in {32, 64, 96,
// 128}) with one workgroup per matrix, 256 to 1024 lanes, so a round's work
// (np (np + 1) / 2 blocks of A, np * d pairs of W, np = n / 2) is a few
// items per lane.  A lives in LDS as NMAX x (NMAX + 1) doubles; W lives in
// LDS too while both fit (NMAX <= 96: 148 KB at 96), else in the workspace
// (L2-resident), where each lane loads all its W pairs of a round (eight)
// before rotating and storing them, so one memory round trip covers a round.  The per-matrix
// descriptors are read from the workspace, so one launch takes any number
// of matrices.
#include <math.h>

#include "launch.hpp"
#include "mr_common.hpp"

namespace mr {

template <int THREADS>
__device__ __forceinline__ double jac_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // red may still be read by a previous reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) r += red[w];  // same order in every lane
  return r;
}

template <typename TA>
__device__ __forceinline__ double jac_ld(const void* A, int64_t idx) {
  return (double)reinterpret_cast<const TA*>(A)[idx];
}

// One rotation of a round: J = [[c, s], [-s, c]] on the index pair (p, q),
// the new diagonal entries, and whether it rotates at all.  One record per
// pair, so a lane needs one LDS address per pair it touches.
struct JacRot {
  double c, s, app, aqq;
  int p, q, rot, pad;
};

template <int NMAX>
struct JacCfg {
  // lanes per workgroup (1024 leaves 128 VGPRs per lane: enough once every
  // pair's rotation is one LDS record, so loop-invariant addresses stay few)
  static constexpr int THREADS = NMAX <= 32 ? 256 : NMAX <= 64 ? 512 : 1024;
  static constexpr bool WLDS = NMAX <= 96;  // eigenvectors in LDS
  static constexpr int LD = NMAX + 1;       // odd row stride of A in LDS
  static constexpr int NP = NMAX / 2;
  static constexpr int PAIRS = (NP * (NP + 1) / 2 + THREADS - 1) / THREADS;  // A blocks per lane
  static constexpr int WPAIRS = (NP * NMAX + THREADS - 1) / THREADS;         // W pairs per lane
  static constexpr int WB = WPAIRS;  // W pairs per memory round trip (all of them)
};

template <typename TA, int NMAX>
__global__ __launch_bounds__(JacCfg<NMAX>::THREADS) void jacobi_kernel(const JacobiLaunch L) {
  using C = JacCfg<NMAX>;
  constexpr int THREADS = C::THREADS, LD = C::LD, NP = C::NP;
  __shared__ double sM[NMAX * LD];
  __shared__ double sW[C::WLDS ? NMAX * NMAX : 1];
  __shared__ JacRot rot_[NP];
  __shared__ double fk[NMAX];
  __shared__ double red[THREADS / 64];

  const JacobiDesc J = L.desc[L.first + blockIdx.x];
  const int tid = threadIdx.x;
  const int d = J.d;
  const int n = d + (d & 1);
  const int np = n / 2;
  const double eps = L.eps;
  double* Wg = J.W;  // global eigenvectors (when they do not fit in LDS)

  // ---- load the symmetric part, trace, finiteness
  double tr = 0.0, nf = 0.0;
  for (int idx = tid; idx < n * n; idx += THREADS) {
    const int i = idx / n, j = idx - (idx / n) * n;
    double v = 0.0;
    if (i < d && j < d) {
      const bool packed = L.a_packed != 0;
      const double a = jac_ld<TA>(J.A, sym_index(i, j, J.lda, d, packed));
      const double at = jac_ld<TA>(J.A, sym_index(j, i, J.lda, d, packed));
      v = 0.5 * (a + at);
      if (!isfinite(v)) nf += 1.0;
      if (i == j) tr += v;
    }
    sM[i * LD + j] = v;
  }
  tr = jac_sum<THREADS>(tr, red);
  nf = jac_sum<THREADS>(nf, red);

  uint32_t flags = 0;
  double s = 1.0;
  if (nf > 0.0 || !isfinite(tr)) flags |= MR_INFO_NONFINITE;
  if (!flags && L.normalize == MR_NORM_TRACE) {
    s = tr;
    if (s == 0.0) flags |= MR_INFO_ZERO_TRACE;
  }

  int sweeps = 0;
  double offnorm = 0.0;
  if (!flags) {
    const double inv_s = 1.0 / s;
    double f2 = 0.0;
    for (int idx = tid; idx < n * n; idx += THREADS) {
      const int i = idx / n, j = idx - (idx / n) * n;
      const double v = sM[i * LD + j] * inv_s;
      sM[i * LD + j] = v;
      f2 += v * v;
    }
    for (int idx = tid; idx < d * d; idx += THREADS) {
      const double e = ((idx / d) == (idx % d)) ? 1.0 : 0.0;
      if (C::WLDS)
        sW[idx] = e;
      else
        Wg[idx] = e;
    }
    f2 = jac_sum<THREADS>(f2, red);  // its barriers also order the sM and W writes before the sweeps
    const double tau = fmax(1e-15 * sqrt(f2), 1e-300);
    // this lane's upper blocks u = tid + THREADS m of the np x np block grid
    int pkr[C::PAIRS], pkc[C::PAIRS];
    {
      const int nblk = np * (np + 1) / 2;
#pragma unroll
      for (int m = 0; m < C::PAIRS; ++m) {
        int u = tid + THREADS * m, kr = 0;
        if (u >= nblk) {
          pkr[m] = -1;
          pkc[m] = 0;
          continue;
        }
        while (u >= np - kr) {  // block row kr holds np - kr upper blocks
          u -= np - kr;
          ++kr;
        }
        pkr[m] = kr;
        pkc[m] = kr + u;
      }
    }
    // this lane's W pairs (k, i) are idx = tid + THREADS m (k = idx / d,
    // i = idx % d): the first one and the uniform step between them, so the
    // rounds walk them without divisions or per-pair registers
    const int wk0 = tid / d, wi0 = tid - (tid / d) * d;
    const int wdk = THREADS / d, wdi = THREADS - (THREADS / d) * d;

    bool rotated_last = true;
    for (int sweep = 0; sweep < L.max_sweeps && rotated_last; ++sweep) {
      int any = 0;
      for (int r = 0; r < n - 1; ++r) {
        int rot = 0;
        if (tid < np) {
          const int k = tid;
          int p, q;
          if (k == 0) {
            p = n - 1;
            q = r;
          } else {
            p = r + k;
            if (p >= n - 1) p -= n - 1;
            q = r - k;
            if (q < 0) q += n - 1;
          }
          if (p > q) {
            const int tmp = p;
            p = q;
            q = tmp;
          }
          const double app = sM[p * LD + p], aqq = sM[q * LD + q], apq = sM[p * LD + q];
          double c = 1.0, sn = 0.0, npp = app, nqq = aqq;
          if (q < d && fabs(apq) > tau) {
            // Rotation that zeroes a_pq (Golub & Van Loan, symmetric Schur 2x2).
            const double theta = (aqq - app) / (2.0 * apq);
            double t;
            if (fabs(theta) > 1e150)
              t = 0.5 / theta;
            else
              t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
            c = 1.0 / sqrt(1.0 + t * t);
            sn = t * c;
            npp = app - t * apq;
            nqq = aqq + t * apq;
            rot = 1;
          }
          rot_[k] = JacRot{c, sn, npp, nqq, p, q, rot, 0};
        }
        if (!__syncthreads_or(rot)) continue;
        any = 1;
        // A <- J^T A J, as independent 2x2 blocks (upper blocks + mirror).
#pragma unroll
        for (int m = 0; m < C::PAIRS; ++m) {
          const int kr = pkr[m], kc = pkc[m];
          if (kr < 0) continue;
          const JacRot& R1 = rot_[kr];
          const JacRot& R2 = rot_[kc];
          if (!R1.rot && !R2.rot) continue;
          const int p1 = R1.p, q1 = R1.q;
          if (kr == kc) {
            sM[p1 * LD + p1] = R1.app;
            sM[q1 * LD + q1] = R1.aqq;
            sM[p1 * LD + q1] = 0.0;
            sM[q1 * LD + p1] = 0.0;
            continue;
          }
          const int p2 = R2.p, q2 = R2.q;
          const double c1 = R1.c, s1 = R1.s, c2 = R2.c, s2 = R2.s;
          const double x00 = sM[p1 * LD + p2], x01 = sM[p1 * LD + q2];
          const double x10 = sM[q1 * LD + p2], x11 = sM[q1 * LD + q2];
          const double y00 = c1 * x00 - s1 * x10, y01 = c1 * x01 - s1 * x11;
          const double y10 = s1 * x00 + c1 * x10, y11 = s1 * x01 + c1 * x11;
          const double z00 = c2 * y00 - s2 * y01, z01 = s2 * y00 + c2 * y01;
          const double z10 = c2 * y10 - s2 * y11, z11 = s2 * y10 + c2 * y11;
          sM[p1 * LD + p2] = z00;
          sM[p1 * LD + q2] = z01;
          sM[q1 * LD + p2] = z10;
          sM[q1 * LD + q2] = z11;
          sM[p2 * LD + p1] = z00;
          sM[q2 * LD + p1] = z01;
          sM[p2 * LD + q1] = z10;
          sM[q2 * LD + q1] = z11;
        }
        // W <- J^T W (rows p, q of W = columns p, q of V), WB pairs of the
        // lane per memory round trip: all of them loaded, then rotated and
        // stored.
        {
          double* Wb = C::WLDS ? sW : Wg;
          int k0 = wk0, i0 = wi0;
          for (int m0 = 0; m0 < C::WPAIRS; m0 += C::WB) {
            double wp[C::WB], wq[C::WB];
            int k = k0, i = i0;
#pragma unroll
            for (int m = 0; m < C::WB; ++m) {
              if (m0 + m < C::WPAIRS && k < np && rot_[k].rot) {
                wp[m] = Wb[rot_[k].p * d + i];
                wq[m] = Wb[rot_[k].q * d + i];
              }
              k += wdk;
              i += wdi;
              if (i >= d) {
                i -= d;
                ++k;
              }
            }
            k = k0;
            i = i0;
#pragma unroll
            for (int m = 0; m < C::WB; ++m) {
              if (m0 + m < C::WPAIRS && k < np && rot_[k].rot) {
                const JacRot& R = rot_[k];
                const double c = R.c, sn = R.s;
                Wb[R.p * d + i] = c * wp[m] - sn * wq[m];
                Wb[R.q * d + i] = sn * wp[m] + c * wq[m];
              }
              k += wdk;
              i += wdi;
              if (i >= d) {
                i -= d;
                ++k;
              }
            }
            k0 = k;
            i0 = i;
          }
        }
        __syncthreads();
      }
      ++sweeps;
      rotated_last = any != 0;
    }
    if (rotated_last) flags |= MR_INFO_NOT_CONVERGED;

    // off-diagonal norm at exit
    double off = 0.0;
    for (int idx = tid; idx < d * d; idx += THREADS) {
      const int i = idx / d, j = idx - (idx / d) * d;
      if (i != j) off += sM[i * LD + j] * sM[i * LD + j];
    }
    offnorm = sqrt(jac_sum<THREADS>(off, red));

    // f_k = (lambda_k + eps)^(-1/4); a non-positive shifted eigenvalue is NOT_PD.
    double bad = 0.0;
    for (int k = tid; k < d; k += THREADS) {
      const double lam = sM[k * LD + k] + eps;
      if (lam > 0.0) {
        fk[k] = sqrt(pow(lam, -0.25));
      } else {
        fk[k] = 0.0;
        bad += 1.0;
      }
    }
    if (jac_sum<THREADS>(bad, red) > 0.0) flags |= MR_INFO_NOT_PD;
  }

  if (!flags || flags == MR_INFO_NOT_CONVERGED) {
    // W' = diag(sqrt f) W into LDS (over A, no longer needed), then
    // X = W'^T W' in 4 x 4 blocks (the sums over k in the same order for
    // (i, j) and (j, i), so X is exactly symmetric).
    for (int idx = tid; idx < d * d; idx += THREADS) {
      const int k = idx / d, i = idx - (idx / d) * d;
      sM[k * LD + i] = fk[k] * (C::WLDS ? sW[idx] : Wg[idx]);
    }
    __syncthreads();
    const int nb4 = (d + 3) / 4;
    for (int blk = tid; blk < nb4 * nb4; blk += THREADS) {
      const int bi = (blk / nb4) * 4, bj = (blk % nb4) * 4;
      double acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
      for (int k = 0; k < d; ++k) {
        double u[4], v[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u[a] = (bi + a < d) ? sM[k * LD + bi + a] : 0.0;
          v[a] = (bj + a < d) ? sM[k * LD + bj + a] : 0.0;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = fma(u[a], v[b], acc[a][b]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (bi + a < d && bj + b < d) J.X[(int64_t)(bi + a) * J.ldx + bj + b] = (float)acc[a][b];
    }
  } else {
    const bool zt = flags == MR_INFO_ZERO_TRACE;
    const float diag = zt ? (float)pow(eps, -0.25) : __builtin_nanf("");
    const float offv = zt ? 0.f : __builtin_nanf("");
    for (int idx = tid; idx < d * d; idx += THREADS) {
      const int i = idx / d, j = idx - (idx / d) * d;
      J.X[(int64_t)i * J.ldx + j] = (i == j) ? diag : offv;
    }
  }

  if (tid == 0) {
    RootState& st = L.state[J.slot];
    st.s = s;
    st.c = 0.0;
    st.out_scale = 0.0;
    st.eps = eps;
    st.d = d;
    st.K = 0;
    st.j = 0;
    st.flags = flags;
    st.residual = (float)offnorm;
    st.method = MR_JACOBI;
    st.sweeps = sweeps;
    st.problem = J.problem;
  }
}

// Descriptor table: the host's records of one batch copied into the workspace.
__global__ __launch_bounds__(64) void jacobi_desc_kernel(const JacobiDescBatch b) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < b.count) b.dst[b.first + i] = b.desc[i];
}

hipError_t launch_jacobi_desc(const JacobiDescBatch& b, hipStream_t s) {
  if (b.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(jacobi_desc_kernel, dim3((b.count + 63) / 64), dim3(64), 0, s, b);
  return hipGetLastError();
}

template <typename TA>
static hipError_t launch_jacobi_t(const JacobiLaunch& L, int nmax, hipStream_t s) {
  switch (nmax) {
    case 32:
      hipLaunchKernelGGL((jacobi_kernel<TA, 32>), dim3(L.count), dim3(JacCfg<32>::THREADS), 0, s, L);
      break;
    case 64:
      hipLaunchKernelGGL((jacobi_kernel<TA, 64>), dim3(L.count), dim3(JacCfg<64>::THREADS), 0, s, L);
      break;
    case 96:
      hipLaunchKernelGGL((jacobi_kernel<TA, 96>), dim3(L.count), dim3(JacCfg<96>::THREADS), 0, s, L);
      break;
    default:
      hipLaunchKernelGGL((jacobi_kernel<TA, 128>), dim3(L.count), dim3(JacCfg<128>::THREADS), 0, s, L);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_jacobi(const JacobiLaunch& L, int nmax, bool a_f64, hipStream_t s) {
  if (L.count <= 0) return hipSuccess;
  return a_f64 ? launch_jacobi_t<double>(L, nmax, s) : launch_jacobi_t<float>(L, nmax, s);
}

}  // namespace mr
