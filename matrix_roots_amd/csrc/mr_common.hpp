// Shared device-side definitions for the gfx950 kernels: vector types, MFMA
// wrappers with their lane layouts, the XCD-aware block remap and the
// upper-triangle tile enumeration.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>
#include <stdint.h>

namespace mr {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Conflict-free LDS store order of the fp16 tile loaders (gemm_core.hpp,
// gemm_h16.hpp); 0 keeps the row-major order.

// Which (row, 16-byte group) of a loader chunk the thread slot idx moves,
// for GPR groups per row and rows padded by one group (row stride
// (GPR + 1) * 16 bytes).  LDS serves 16-byte accesses 16 lanes per cycle
// over 64 four-byte banks, so a cycle's 16 lanes cover 16 / GPR rows whose
// GPR * 4-bank spans should be disjoint.  Row-major slots put adjacent rows
// in one cycle, which overlap (rows r and r+3 for GPR = 4, r and r+1 for
// GPR = 8); rows 4 apart (GPR = 4: stride 20 banks, spans start 0, 16, 32,
// 48) or 8 apart (GPR = 8: stride 36 banks, spans start 0 and 32) do not.
// Each row's GPR groups still come from consecutive lanes.
template <int GPR>
__device__ __forceinline__ void tile_slot(int idx, int& row, int& grp) {
  if constexpr (GPR == 4) {
    const int g = idx >> 4, q = idx & 15;
    row = 16 * (g >> 2) + (g & 3) + 4 * (q >> 2);
    grp = q & 3;
    return;
  } else if constexpr (GPR == 8) {
    const int g = idx >> 4, q = idx & 15;
    row = 16 * (g >> 3) + (g & 7) + 8 * (q >> 3);
    grp = q & 7;
    return;
  }
  row = idx / GPR;
  grp = idx % GPR;
}
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

// --------------------------------------------------------------------------
// MFMA lane layouts (verified on gfx950 with an in-bounds probe):
//
// v_mfma_f32_32x32x2_f32, D(32x32) += A(32x2) B(2x32):
//   lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32];
//   D value v (0..15) of lane l is D[8*(v/4) + 4*(l/32) + v%4][l % 32].
// v_mfma_f32_32x32x16_f16, D(32x32) += A(32x16) B(16x32):
//   lane l supplies A[l % 32][8*(l/32) + e] and B[8*(l/32) + e][l % 32],
//   e = 0..7; D is laid out as for v_mfma_f32_32x32x2_f32.
// v_mfma_f64_16x16x4_f64, D(16x16) += A(16x4) B(4x16):
//   lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
//   D value v (0..3) of lane l is D[4*v + l/16][l % 16].
// --------------------------------------------------------------------------
__device__ __forceinline__ v16f mfma_f32_32x32x2(float a, float b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16_32x32x16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4d mfma_f64_16x16x4(double a, double b, v4d c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int f32_row(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int f64_row(int lane, int v) { return 4 * v + (lane >> 4); }

// Workgroup b of a 1-D grid lands on XCD b % 8.  Within a range of n blocks
// that starts on a multiple of 8, renumber so that each XCD receives one
// contiguous run of logical blocks: neighbouring tiles of one matrix (which
// share operand panels) then share that XCD's L2.  Launches remap each job or
// size class separately (8-aligned, padded), so every XCD gets the same mix of
// cheap and expensive tiles.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n) {
  const int64_t per = n / kNumXcd;
  const int64_t full = per * kNumXcd;
  if (b >= full) return b;  // ragged remainder keeps its order
  return (b % kNumXcd) * per + b / kNumXcd;
}

// Offset of element (i, j) of a symmetric d x d matrix stored full
// (row-major, leading dimension ld) or packed (upper triangle by rows:
// (i, j), i <= j, at i d - i (i - 1) / 2 + j - i); a lower element of a
// packed matrix reads its mirror.
__host__ __device__ __forceinline__ int64_t sym_index(int64_t i, int64_t j, int64_t ld, int64_t d, bool packed) {
  if (!packed) return i * ld + j;
  if (i > j) {
    const int64_t t = i;
    i = j;
    j = t;
  }
  return i * d - (i * (i - 1)) / 2 + (j - i);
}

// Tile (bi, bj) of 32 x 32 of the symmetric part (A + A^T)/2 through LDS
// (256 threads, 4 rows each).  Full storage: tiles (bi, bj) into ta and
// (bj, bi) into tb, both read along rows.  Packed storage: the upper tile of
// the pair into ta (its rows are contiguous); the matrix is symmetric by
// construction, so its symmetric part is the stored value itself.
template <typename TA>
__device__ __forceinline__ void load_sym_tile(const void* A, int64_t lda, int d, bool packed, int bi, int bj,
                                              double (*ta)[33], double (*tb)[33]) {
  const TA* a = reinterpret_cast<const TA*>(A);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (packed) {
    const int ui = bi < bj ? bi : bj, uj = bi < bj ? bj : bi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = ty + 8 * e;
      const int gi = ui * 32 + r, gj = uj * 32 + tx;
      ta[r][tx] = (gi < d && gj < d) ? (double)a[sym_index(gi, gj, 0, d, true)] : 0.0;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = ty + 8 * e;
      const int gi = bi * 32 + r, gj = bj * 32 + tx;
      ta[r][tx] = (gi < d && gj < d) ? (double)a[(int64_t)gi * lda + gj] : 0.0;
      const int hi = bj * 32 + r, hj = bi * 32 + tx;
      tb[r][tx] = (hi < d && hj < d) ? (double)a[(int64_t)hi * lda + hj] : 0.0;
    }
  }
  __syncthreads();
}
// Tile pair u of the upper triangle of a T x T grid of tiles, row by row:
// (bi, bj) with bi <= bj, row i holding T - i pairs (the first at
// i T - i (i - 1) / 2).  A workgroup that owns the pair reads tiles (bi, bj)
// and (bj, bi) once and writes both.
__host__ __device__ __forceinline__ void upper_pair(int u, int T, int& bi, int& bj) {
  auto first = [T](int k) { return k * T - k * (k - 1) / 2; };
  const double b = 2.0 * T + 1.0;
  int i = (int)(0.5 * (b - sqrt(b * b - 8.0 * u)));
  if (i < 0) i = 0;
  while (i > 0 && first(i) > u) --i;
  while (first(i + 1) <= u) ++i;
  bi = i;
  bj = i + (u - first(i));
}

// Element (r, c) of the tile loaded by load_sym_tile.
__device__ __forceinline__ double sym_tile_value(bool packed, int bi, int bj, int r, int c, const double (*ta)[33],
                                                 const double (*tb)[33]) {
  if (packed) return bi <= bj ? ta[r][c] : ta[c][r];
  return 0.5 * (ta[r][c] + tb[c][r]);
}

// Direct global -> LDS copies (global_load_lds_dwordx4: 16 bytes per lane
// into 1 KB of consecutive LDS per instruction).  Operand chunks of UPR
// 16-byte units per row sit unpadded, the unit of k-group kg of row r in slot
// dl_slot(r, kg, UPR) (an involution in kg), so the 16 lanes of one 128-bit
// LDS read cycle (16 consecutive rows, one k-group) hit 16 distinct bank
// groups.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ int dl_slot(int row, int kg, int upr) { return kg ^ ((row / (16 / upr)) % upr); }

// A pointer every lane of the wave holds (a workgroup's operand base) as a
// scalar value, opaque to the compiler: the direct-to-LDS copies then take it
// as their scalar base with a 32-bit lane offset, instead of a 64-bit address
// per lane that the compiler would hoist out of the main loop.
__device__ __forceinline__ const char* wave_uniform(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  const char* u = reinterpret_cast<const char*>(lo | (hi << 32));
  asm volatile("" : "+s"(u));
  return u;
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until every LDS (and scalar memory) operation of this wave is done.
__device__ __forceinline__ void wait_lgkmcnt0() {
  // vmcnt [3:0] and [15:14] and expcnt [6:4] at their maxima, lgkmcnt [11:8] = 0
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// L2-friendly tile orders.  A launch keeps ~64 output tiles per XCD in
// flight (32 CUs x 2 workgroups), and tiles advance through K at the same
// pace, so what decides the operand traffic is how many distinct operand
// panels one window of consecutive tiles touches.  Row-major order over a
// 32-tile-wide grid touches ~2 row panels and ~32 column panels per window
// (each column panel chunk used about twice before it leaves L2); bands of
// G tile rows walked column by column touch ~G + G panels per G*G tiles.
// G = 1 is the row-major order.
constexpr int kTileGroup = 8;

// Tile u of the upper triangle (ti <= tj) of a T x T grid, in bands of
// kTileGroup tile rows, each band column by column.
__host__ __device__ __forceinline__ void upper_tile_grouped(int u, int T, int& ti, int& tj) {
  constexpr int G = kTileGroup;
  int b0 = 0;
  while (true) {
    const int h = T - b0 < G ? T - b0 : G;
    const int tri = h * (h + 1) / 2;  // columns b0 .. b0+h-1 hold 1 .. h tiles of the band
    const int total = tri + (T - b0 - h) * h;
    if (u < total) {
      if (u < tri) {
        int c = 0;
        while ((c + 1) * (c + 2) / 2 <= u) ++c;
        tj = b0 + c;
        ti = b0 + (u - c * (c + 1) / 2);
      } else {
        const int v = u - tri;
        tj = b0 + h + v / h;
        ti = b0 + v % h;
      }
      return;
    }
    u -= total;
    b0 += G;
  }
}

// Tile u of a full TM x TN grid, in bands of kTileGroup tile rows, each
// band column by column.
__device__ __forceinline__ void full_tile_grouped(int u, int TM, int TN, int& ti, int& tj) {
  constexpr int G = kTileGroup;
  const int b0 = (u / (G * TN)) * G;
  const int h = TM - b0 < G ? TM - b0 : G;
  const int v = u - b0 * TN;
  tj = v / h;
  ti = b0 + v % h;
}

// Upper-triangle tile u (row-major over ti <= tj) of a T x T tile grid.
__device__ __forceinline__ void upper_tile(int u, int T, int& ti, int& tj) {
  // rows ti hold T - ti tiles; walk the rows (T <= 128 in practice).
  int r = 0;
  int rem = u;
  while (rem >= T - r) {
    rem -= T - r;
    ++r;
  }
  ti = r;
  tj = r + rem;
}

}  // namespace mr
