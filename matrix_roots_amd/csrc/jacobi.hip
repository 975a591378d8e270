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
// rows of W = V^T in the workspace (float64).  Then, with
// f_k = (lambda_k + eps)^(-1/4), X = sum_k f_k v_k v_k^T is formed as
// W'^T W' with W' = diag(sqrt f) W in LDS, which is exactly symmetric.
// Odd d is padded with a zero row and column that never rotates.
#include <math.h>

#include "launch.hpp"
#include "mr_common.hpp"

namespace mr {

constexpr int kJN = kJacobiMaxD;       // max padded size
constexpr int kJLD = kJacobiMaxD + 1;  // LDS row stride (odd: spreads banks)

__device__ __forceinline__ double jac_sum(double v, double* red) {
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

template <typename TA>
__device__ __forceinline__ double jac_ld(const void* A, int64_t idx) {
  return (double)reinterpret_cast<const TA*>(A)[idx];
}

constexpr int kWBatch = 8;  // eigenvector element pairs per thread per memory round trip
// Upper pairs (kr <= kc) of the rotations of one round, per thread: the
// assignment is fixed for the whole kernel, so it is computed once and not
// by integer divisions in every round.
constexpr int kPairsPerThread = ((kJN / 2) * (kJN / 2 + 1) / 2 + 255) / 256;

template <typename TA>
__global__ __launch_bounds__(256) void jacobi_kernel(const JacobiBatch B) {
  __shared__ double sM[kJN * kJLD];
  __shared__ double rc[kJN / 2], rs[kJN / 2], rpp[kJN / 2], rqq[kJN / 2];
  __shared__ int rp[kJN / 2], rq[kJN / 2], rrot[kJN / 2];
  __shared__ double fk[kJN];
  __shared__ double red[256];

  const JacobiJob& J = B.job[blockIdx.x];
  const int tid = threadIdx.x;
  const int d = J.d;
  const int n = d + (d & 1);
  const int np = n / 2;
  const double eps = B.eps;
  double* W = J.W;

  // ---- load the symmetric part, trace, finiteness
  double tr = 0.0, nf = 0.0;
  for (int idx = tid; idx < n * n; idx += 256) {
    const int i = idx / n, j = idx % n;
    double v = 0.0;
    if (i < d && j < d) {
      const bool packed = B.a_packed != 0;
      const double a = jac_ld<TA>(J.A, sym_index(i, j, J.lda, d, packed));
      const double at = jac_ld<TA>(J.A, sym_index(j, i, J.lda, d, packed));
      v = 0.5 * (a + at);
      if (!isfinite(v)) nf += 1.0;
      if (i == j) tr += v;
    }
    sM[i * kJLD + j] = v;
  }
  tr = jac_sum(tr, red);
  nf = jac_sum(nf, red);

  uint32_t flags = 0;
  double s = 1.0;
  if (nf > 0.0 || !isfinite(tr)) flags |= MR_INFO_NONFINITE;
  if (!flags && B.normalize == MR_NORM_TRACE) {
    s = tr;
    if (s == 0.0) flags |= MR_INFO_ZERO_TRACE;
  }

  int sweeps = 0;
  double offnorm = 0.0;
  if (!flags) {
    const double inv_s = 1.0 / s;
    double f2 = 0.0;
    for (int idx = tid; idx < n * n; idx += 256) {
      const int i = idx / n, j = idx % n;
      const double v = sM[i * kJLD + j] * inv_s;
      sM[i * kJLD + j] = v;
      f2 += v * v;
    }
    for (int idx = tid; idx < d * d; idx += 256) W[idx] = ((idx / d) == (idx % d)) ? 1.0 : 0.0;
    f2 = jac_sum(f2, red);  // also orders the W and sM writes before the sweeps
    const double tau = fmax(1e-15 * sqrt(f2), 1e-300);
    // this thread's upper pairs u = tid + 256 m of the np x np rotation grid
    int pkr[kPairsPerThread], pkc[kPairsPerThread];
    {
      const int npairs = np * (np + 1) / 2;
#pragma unroll
      for (int m = 0; m < kPairsPerThread; ++m) {
        int u = tid + 256 * m, kr = 0;
        if (u >= npairs) {
          pkr[m] = -1;
          pkc[m] = 0;
          continue;
        }
        while (u >= np - kr) {  // row kr holds np - kr upper pairs
          u -= np - kr;
          ++kr;
        }
        pkr[m] = kr;
        pkc[m] = kr + u;
      }
    }
    // the first of this thread's (k, i) eigenvector pairs idx = tid + 256 m
    // and the step between consecutive ones, without divisions in the rounds
    const int wk0 = tid / d, wi0 = tid % d, wdk = 256 / d, wdi = 256 % d;

    bool rotated_last = true;
    for (int sweep = 0; sweep < B.max_sweeps && rotated_last; ++sweep) {
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
            p = (r + k) % (n - 1);
            q = (r - k + n - 1) % (n - 1);
          }
          if (p > q) {
            const int tmp = p;
            p = q;
            q = tmp;
          }
          const double app = sM[p * kJLD + p], aqq = sM[q * kJLD + q], apq = sM[p * kJLD + q];
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
          rc[k] = c;
          rs[k] = sn;
          rpp[k] = npp;
          rqq[k] = nqq;
          rp[k] = p;
          rq[k] = q;
          rrot[k] = rot;
        }
        if (!__syncthreads_or(rot)) continue;
        any = 1;
        // A <- J^T A J, as independent 2x2 blocks (upper blocks + mirror).
#pragma unroll
        for (int m = 0; m < kPairsPerThread; ++m) {
          const int kr = pkr[m], kc = pkc[m];
          if (kr < 0) continue;
          const int rot1 = rrot[kr], rot2 = rrot[kc];
          if (!rot1 && !rot2) continue;
          const int p1 = rp[kr], q1 = rq[kr];
          if (kr == kc) {
            sM[p1 * kJLD + p1] = rpp[kr];
            sM[q1 * kJLD + q1] = rqq[kr];
            sM[p1 * kJLD + q1] = 0.0;
            sM[q1 * kJLD + p1] = 0.0;
            continue;
          }
          const int p2 = rp[kc], q2 = rq[kc];
          const double c1 = rc[kr], s1 = rs[kr], c2 = rc[kc], s2 = rs[kc];
          const double x00 = sM[p1 * kJLD + p2], x01 = sM[p1 * kJLD + q2];
          const double x10 = sM[q1 * kJLD + p2], x11 = sM[q1 * kJLD + q2];
          const double y00 = c1 * x00 - s1 * x10, y01 = c1 * x01 - s1 * x11;
          const double y10 = s1 * x00 + c1 * x10, y11 = s1 * x01 + c1 * x11;
          const double z00 = c2 * y00 - s2 * y01, z01 = s2 * y00 + c2 * y01;
          const double z10 = c2 * y10 - s2 * y11, z11 = s2 * y10 + c2 * y11;
          sM[p1 * kJLD + p2] = z00;
          sM[p1 * kJLD + q2] = z01;
          sM[q1 * kJLD + p2] = z10;
          sM[q1 * kJLD + q2] = z11;
          sM[p2 * kJLD + p1] = z00;
          sM[q2 * kJLD + p1] = z01;
          sM[p2 * kJLD + q1] = z10;
          sM[q2 * kJLD + q1] = z11;
        }
        // W <- J^T W (rows p, q of W = columns p, q of V).  W lives in global
        // memory: each thread first loads kWBatch element pairs, then
        // rotates and stores them, so one memory latency covers the batch
        // instead of one per pair.
        int wk = wk0, wi = wi0;
        for (int base = tid; base < np * d; base += 256 * kWBatch) {
          double wp[kWBatch], wq[kWBatch];
          int64_t op[kWBatch], oq[kWBatch];
          int kk[kWBatch];
#pragma unroll
          for (int u = 0; u < kWBatch; ++u) {
            const int k = wk, i = wi;  // (k, i) of idx = base + 256 u
            wk += wdk;
            wi += wdi;
            if (wi >= d) {
              wi -= d;
              ++wk;
            }
            kk[u] = -1;
            if (k < np && rrot[k]) {
              kk[u] = k;
              op[u] = (int64_t)rp[k] * d + i;
              oq[u] = (int64_t)rq[k] * d + i;
              wp[u] = W[op[u]];
              wq[u] = W[oq[u]];
            }
          }
#pragma unroll
          for (int u = 0; u < kWBatch; ++u) {
            if (kk[u] < 0) continue;
            const double c = rc[kk[u]], sn = rs[kk[u]];
            W[op[u]] = c * wp[u] - sn * wq[u];
            W[oq[u]] = sn * wp[u] + c * wq[u];
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
    for (int idx = tid; idx < d * d; idx += 256) {
      const int i = idx / d, j = idx % d;
      if (i != j) off += sM[i * kJLD + j] * sM[i * kJLD + j];
    }
    offnorm = sqrt(jac_sum(off, red));

    // f_k = (lambda_k + eps)^(-1/4); a non-positive shifted eigenvalue is NOT_PD.
    double bad = 0.0;
    for (int k = tid; k < d; k += 256) {
      const double lam = sM[k * kJLD + k] + eps;
      if (lam > 0.0) {
        fk[k] = sqrt(pow(lam, -0.25));
      } else {
        fk[k] = 0.0;
        bad += 1.0;
      }
    }
    if (jac_sum(bad, red) > 0.0) flags |= MR_INFO_NOT_PD;
  }

  if (!flags || flags == MR_INFO_NOT_CONVERGED) {
    // W' = diag(sqrt f) W into LDS, then X = W'^T W' in 8 x 8 blocks.
    for (int idx = tid; idx < d * d; idx += 256) {
      const int k = idx / d, i = idx % d;
      sM[k * kJLD + i] = fk[k] * W[(int64_t)k * d + i];
    }
    __syncthreads();
    const int nb8 = (d + 7) / 8;
    for (int blk = tid; blk < nb8 * nb8; blk += 256) {
      const int bi = (blk / nb8) * 8, bj = (blk % nb8) * 8;
      double acc[8][8];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
      for (int k = 0; k < d; ++k) {
        double u[8], v[8];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          u[a] = (bi + a < d) ? sM[k * kJLD + bi + a] : 0.0;
          v[a] = (bj + a < d) ? sM[k * kJLD + bj + a] : 0.0;
        }
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int b = 0; b < 8; ++b) acc[a][b] = fma(u[a], v[b], acc[a][b]);
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b)
          if (bi + a < d && bj + b < d) J.X[(int64_t)(bi + a) * J.ldx + bj + b] = (float)acc[a][b];
    }
  } else {
    const bool zt = flags == MR_INFO_ZERO_TRACE;
    const float diag = zt ? (float)pow(eps, -0.25) : __builtin_nanf("");
    const float off = zt ? 0.f : __builtin_nanf("");
    for (int idx = tid; idx < d * d; idx += 256) {
      const int i = idx / d, j = idx % d;
      J.X[(int64_t)i * J.ldx + j] = (i == j) ? diag : off;
    }
  }

  if (tid == 0) {
    RootState& st = B.state[J.slot];
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

hipError_t launch_jacobi(const JacobiBatch& b, hipStream_t s) {
  if (b.njobs <= 0) return hipSuccess;
  if (b.a_f64)
    hipLaunchKernelGGL(jacobi_kernel<double>, dim3(b.njobs), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL(jacobi_kernel<float>, dim3(b.njobs), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace mr
