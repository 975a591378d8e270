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
// swizzled by dl_slot) in three stages of 48 KiB, the copies of chunk c + 2
// spread over chunk c's products; one barrier per chunk.
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

// Copy j (0 .. 5) of chunk k0 .. k0+31 of rows m0.. (A) and n0.. (B) into
// `stage`, which holds 12 arrays of 256 units (A planes 0 .. 5, then B
// planes): wave w copies units 64 (w & 3) .. +63 of array 2 j + (w >> 2), an
// A plane for j < 3, a B plane after.  The address is a wave-uniform base
// (the plane at row m0 or n0, column k0) plus a 32-bit lane offset within the
// tile's 128 rows, so each copy is one instruction on a scalar base.
__device__ __forceinline__ void oz_copy(const OzPlanes& A, const OzPlanes& B, int64_t ld, int m0, int n0, int k0,
                                        unsigned char* stage, int wave, int lane, int j) {
  const int base_u = (wave & 3) * 64;
  const int u = base_u + lane;
  const int row = u / OzCfg::UPR;
  const int kg = dl_slot(row, u % OzCfg::UPR, OzCfg::UPR);  // the map is its own inverse
  const bool is_a = j < OzCfg::S / 2;
  uint32_t off = (uint32_t)row * (uint32_t)ld + (uint32_t)(kg * 16);
  const int a = 2 * j + (wave >> 2);
  const int p = is_a ? a : a - OzCfg::S;
  // (p depends on the wave: select the pointer, never index the lists with it)
  const int8_t* P = nullptr;
#pragma unroll
  for (int q = 0; q < OzCfg::S; ++q)
    if (q == p) P = is_a ? A.p[q] : B.p[q];
  const char* base = wave_uniform(P + (int64_t)(is_a ? m0 : n0) * ld + k0);
  asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
  __builtin_amdgcn_global_load_lds((global_void_ptr)(base + off),
                                   (lds_void_ptr)(stage + (a * OzCfg::PLANE_UNITS + base_u) * 16), 16, 0, 0);
}

// The whole chunk k0 .. k0+31 into `stage`.
__device__ __forceinline__ void oz_issue(const OzPlanes& A, const OzPlanes& B, int64_t ld, int m0, int n0, int k0,
                                         unsigned char* stage, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < OzCfg::S; ++j) oz_copy(A, B, ld, m0, n0, k0, stage, wave, lane, j);
}

// Fragment (row r, k-group kg) of array `plane` of a stage.
__device__ __forceinline__ v4i oz_frag(const unsigned char* __restrict__ st, int plane, int r, int kg) {
  return *reinterpret_cast<const v4i*>(st + (plane * OzCfg::PLANE_UNITS + r * OzCfg::UPR + dl_slot(r, kg, OzCfg::UPR)) *
                                                16);
}

// The copies a chunk's products carry for a later chunk.
struct OzNext {
  bool on;
  int k0;
  unsigned char* stage;
};

// acc[r][cb] += sum_{p + q = r} D^A_p D^B_q^T over one chunk, B plane by B
// plane (q = 0 .. 5 pairs with A planes 0 .. 5 - q).  The B fragments of
// plane q + 1 are read while the products of plane q run (two register
// sets), each wait falls on reads issued a group of products earlier, and
// copy q of the next chunk goes out with group q; scheduling barriers keep
// that order.
__device__ __forceinline__ void oz_chunk(const unsigned char* __restrict__ st, v16i (&acc)[kOzSlices][2], int lane,
                                         int wave, const OzPlanes& A, const OzPlanes& B, int64_t ld, int m0, int n0,
                                         const OzNext& next) {
  const int kg = lane >> 5;
  const int ra = (wave >> 1) * 32 + (lane & 31);
  const int rb = (wave & 1) * 64 + (lane & 31);
  v4i af[OzCfg::S];
  v4i bf[2][2];
  af[0] = oz_frag(st, 0, ra, kg);
  bf[0][0] = oz_frag(st, OzCfg::S, rb, kg);
  bf[0][1] = oz_frag(st, OzCfg::S, rb + 32, kg);
#pragma unroll
  for (int p = 1; p < OzCfg::S; ++p) af[p] = oz_frag(st, p, ra, kg);
#pragma unroll
  for (int q = 0; q < OzCfg::S; ++q) {
    // B plane q (before q = 0 also the A planes) is the only read in
    // flight: wait for it before issuing plane q + 1's
    wait_lgkmcnt0();
    if (q + 1 < OzCfg::S) {
      bf[(q + 1) & 1][0] = oz_frag(st, OzCfg::S + q + 1, rb, kg);
      bf[(q + 1) & 1][1] = oz_frag(st, OzCfg::S + q + 1, rb + 32, kg);
    }
    if (next.on) oz_copy(A, B, ld, m0, n0, next.k0, next.stage, wave, lane, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p + q < OzCfg::S; ++p)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[p + q][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[p], bf[q & 1][cb], acc[p + q][cb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Accumulators of the 128 x 128 tile at (m0, n0) of A B^T over K (a multiple
// of 32; rows m0 .. m0+127 and n0 .. n0+127 exist in both plane sets).  Ends
// with a block barrier: the LDS is free for the epilogue.
__device__ __forceinline__ void oz_nt_tile(const OzPlanes& A, const OzPlanes& B, int64_t ld, int K, int m0, int n0,
                                           unsigned char* __restrict__ lds, v16i (&acc)[kOzSlices][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
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
    // chunk c + 2 goes into the stage chunk c - 1 occupied
    const OzNext next{c + 2 < nch, (c + 2) * OzCfg::BK, lds + ((c + 2) % OzCfg::NST) * OzCfg::STAGE_BYTES};
    oz_chunk(st, acc, lane, wave, A, B, ld, m0, n0, next);
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
