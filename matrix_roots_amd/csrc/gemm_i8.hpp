// Float64-accurate products on the int8 matrix cores (int8 digit slices).
//
// A float64 matrix X with one power-of-two exponent per row, e_i >= log2
// max_j |X_ij|, is held as kOzSlices int8 digit planes D_0 .. D_5:
//
//   X_ij ~= 2^e_i * sum_p D_p[i][j] 2^-(6 + 7 p),   |D_p[i][j]| <= 65,
//
// the balanced base-128 digits of X_ij rounded to a multiple of 2^(e_i - 41),
// so the planes hold X to 2^(e_i - 42).  The NT product C = A B^T of
// two such matrices is
//
//   C_ij = 2^(eA_i + eB_j - 12) * sum_r 2^(-7 r) * (sum_{p + q = r} D^A_p D^B_q^T)_ij,
//
// with every plane product D^A_p D^B_q^T exact in int32 on
// v_mfma_i32_32x32x32_i8 (|sum| <= 6 * K * 65^2 < 2^31 for K < 84000), one
// int32 accumulator per anti-diagonal r = p + q, and the pairs with
// p + q > 5 left out: they weigh at most 2^-47 relative to the leading one,
// below the representation error of the planes.  That is 21 int8 products
// per float64 product.  The scheme is the error-free splitting of matrix
// products into exactly computable slices of Ozaki, Ogita, Oishi and Rump
// (Numerical Algorithms 59, 2012), with the integer slices and integer
// accumulation of Ootomo, Ozaki and Yokota ("DGEMM on integer matrix
// multiplication unit", IJHPCA 2024); the digit form, the truncation and the
// accumulation per anti-diagonal are this file's.
//
// Planes are row-major with row stride dp = d rounded up to 128 (rows and
// columns past d hold zero digits); each plane is contiguous, the six of a
// matrix need not be (OzPlanes lists them).
#pragma once

#include "launch.hpp"
#include "mr_common.hpp"

namespace mr {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct OzPlanes {
  int8_t* p[kOzSlices];
};

// Digit planes of value v with exponent e (|v| <= 2^e up to rounding):
// N = rint(v 2^(41 - e)) in two int32 halves (N = hi 2^21 + lo, both exact
// conversions of float64), then balanced base-128 digits from the least
// significant, each in [-64, 63] with the carry passed up; the leading digit
// takes what is left (|digit| <= 65), clamped to the int8 range, which only
// an input outside the bound (an indefinite matrix, a failed iteration) can
// reach.  Digit p has weight 2^(e - 6 - 7 p).
__host__ __device__ __forceinline__ void oz_digits(double v, int e, int8_t (&dg)[kOzSlices]) {
  static_assert(kOzSlices == 6, "three digits per int32 half");
  const double t = fmin(fmax(ldexp(v, 20 - e), -1073741824.0), 1073741824.0);
  const double th = rint(t);
  int hi = (int)th;
  int x = (int)rint(ldexp(t - th, 21));  // |x| <= 2^20
#pragma unroll
  for (int p = kOzSlices - 1; p >= 3; --p) {
    const int dd = ((x + 64) & 127) - 64;
    dg[p] = (int8_t)dd;
    x = (x - dd) >> 7;
  }
  hi += x;
#pragma unroll
  for (int p = 2; p >= 1; --p) {
    const int dd = ((hi + 64) & 127) - 64;
    dg[p] = (int8_t)dd;
    hi = (hi - dd) >> 7;
  }
  dg[0] = (int8_t)min(max(hi, -127), 127);
}

// 128 x 128 output tile, 512 threads = 8 waves in a 4 x 2 grid of 32 x 64
// (one 32 x 32 MFMA block per row of waves, two per column), six int32
// accumulators of 32 x 64 per wave (192 registers: two waves per SIMD).
// K-chunks of 32 digits per plane, copied straight to LDS (16-byte units,
// swizzled by dl_slot) in three stages of 48 KiB; one barrier per chunk.
struct OzCfg {
  static constexpr int S = kOzSlices;
  static constexpr int BM = kOzTile, BN = kOzTile, BK = 32, UPR = BK / 16;
  static constexpr int THREADS = 512;
  static constexpr int PLANE_UNITS = BM * UPR;                  // 16-byte units per plane and operand
  static constexpr int STAGE_BYTES = 2 * S * PLANE_UNITS * 16;  // A planes then B planes
  static constexpr int NST = 3;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int PAIRS = S * (S + 1) / 2;
};
static_assert(OzCfg::S * 2 * OzCfg::PLANE_UNITS == OzCfg::THREADS * OzCfg::S, "one unit per thread and plane pair");

// Copy chunk k0 .. k0+31 of rows m0.. (A) and n0.. (B), every plane, into
// `stage`: 12 arrays of 256 units; wave w copies units 64 (w & 3) .. +63 of
// the arrays of parity w >> 2.
__device__ __forceinline__ void oz_issue(const OzPlanes& A, const OzPlanes& B, int64_t ld, int m0, int n0, int k0,
                                         unsigned char* stage, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < OzCfg::S; ++j) {
    const int a = 2 * j + (wave >> 2);
    const int op = a / OzCfg::S, p = a % OzCfg::S;
    // (p depends on the wave: select the pointer, never index the lists with it)
    const int8_t* P = nullptr;
#pragma unroll
    for (int q = 0; q < OzCfg::S; ++q)
      if (q == p) P = op == 0 ? A.p[q] : B.p[q];
    const int r0 = op == 0 ? m0 : n0;
    const int base_u = (wave & 3) * 64;
    const int u = base_u + lane;
    const int row = u / OzCfg::UPR;
    const int kg = dl_slot(row, u % OzCfg::UPR, OzCfg::UPR);  // the map is its own inverse
    const int8_t* src = P + (int64_t)(r0 + row) * ld + k0 + kg * 16;
    __builtin_amdgcn_global_load_lds((global_void_ptr)src,
                                     (lds_void_ptr)(stage + (a * OzCfg::PLANE_UNITS + base_u) * 16), 16, 0, 0);
  }
}

// acc[r][cb] += sum_{p + q = r} D^A_p D^B_q^T over one chunk.
__device__ __forceinline__ void oz_chunk(const unsigned char* __restrict__ st, v16i (&acc)[kOzSlices][2], int lane,
                                         int wm, int wn) {
  const int kg = lane >> 5;
  v4i af[OzCfg::S];
#pragma unroll
  for (int p = 0; p < OzCfg::S; ++p) {
    const int r = wm * 32 + (lane & 31);
    af[p] = *reinterpret_cast<const v4i*>(
        st + (p * OzCfg::PLANE_UNITS + r * OzCfg::UPR + dl_slot(r, kg, OzCfg::UPR)) * 16);
  }
#pragma unroll
  for (int q = 0; q < OzCfg::S; ++q) {
    v4i bf[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = wn * 64 + cb * 32 + (lane & 31);
      bf[cb] = *reinterpret_cast<const v4i*>(
          st + ((OzCfg::S + q) * OzCfg::PLANE_UNITS + r * OzCfg::UPR + dl_slot(r, kg, OzCfg::UPR)) * 16);
    }
#pragma unroll
    for (int p = 0; p + q < OzCfg::S; ++p)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[p + q][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[p], bf[cb], acc[p + q][cb], 0, 0, 0);
  }
}

// Accumulators of the 128 x 128 tile at (m0, n0) of A B^T over K (a multiple
// of 32; rows m0 .. m0+127 and n0 .. n0+127 exist in both plane sets).  Ends
// with a block barrier: the LDS is free for the epilogue.
__device__ __forceinline__ void oz_nt_tile(const OzPlanes& A, const OzPlanes& B, int64_t ld, int K, int m0, int n0,
                                           unsigned char* __restrict__ lds, v16i (&acc)[kOzSlices][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int r = 0; r < OzCfg::S; ++r)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[r][cb][v] = 0;
  const int nch = K / OzCfg::BK;
  if (nch > 0) oz_issue(A, B, ld, m0, n0, 0, lds, wave, lane);
  if (nch > 1) oz_issue(A, B, ld, m0, n0, OzCfg::BK, lds + OzCfg::STAGE_BYTES, wave, lane);
  for (int c = 0; c < nch; ++c) {
    const unsigned char* st = lds + (c % OzCfg::NST) * OzCfg::STAGE_BYTES;
    // chunk c is complete once at most the next chunk's copies are in flight
    if (c + 1 < nch)
      wait_vmcnt<OzCfg::S>();
    else
      wait_vmcnt<0>();
    wait_lgkmcnt0();  // this wave's reads of chunk c - 1 have returned
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // chunk c visible to all waves; all are done with chunk c - 1
    asm volatile("" ::: "memory");
    if (c + 2 < nch)  // into the stage chunk c - 1 occupied
      oz_issue(A, B, ld, m0, n0, (c + 2) * OzCfg::BK, lds + ((c + 2) % OzCfg::NST) * OzCfg::STAGE_BYTES, wave, lane);
    oz_chunk(st, acc, lane, wm, wn);
  }
  __syncthreads();  // no wave reuses the LDS while another may still read the last stage
}

// float64 value of element v of block cb: sum_r 2^(-7 r) acc[r], times
// 2^(e - 12) for the caller's e = eA_i + eB_j (e = 12: the unscaled sum).
__device__ __forceinline__ double oz_value(const v16i (&acc)[kOzSlices][2], int cb, int v, int e) {
  double x = (double)acc[kOzSlices - 1][cb][v];
#pragma unroll
  for (int r = kOzSlices - 2; r >= 0; --r) x = x * (1.0 / 128.0) + (double)acc[r][cb][v];
  return ldexp(x, e - 12);
}

}  // namespace mr
