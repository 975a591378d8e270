// Wide-store epilogue for the 32 x 32 MFMA accumulator layout.
//
// A lane of a 32 x 32 block holds one column and 16 rows, so storing straight
// from the accumulators issues 2-byte stores (split fp16 outputs) that cover
// 64 bytes per row: the store and a_k-term load instructions then dominate
// kernels whose contraction is short.  Instead, each wave moves a 64-row
// slab of its sub-tile (2 x 2 blocks of 32 x 32) into a private, padded LDS
// slab and reads it back twice:
//   * by rows, 8 consecutive columns per lane: 16-byte loads of the a_k term
//     and 16-byte stores of the output row chunk (the final value is written
//     back into the slab);
//   * by columns, 8 consecutive rows per lane: 16-byte stores of the
//     transposed (or mirrored) output.
// Eight lanes cover the 64 rows of one output column, so a transposed store
// instruction writes 128-byte row segments.  Padding of 4 floats per
// 64-float row keeps the slab writes (32 lanes per row) and the row-chunk
// reads (16 lanes over two rows) free of bank conflicts; the column reads
// (4-byte, eight rows apart) see four-way conflicts, which cost far less than
// the global stores they feed.  The slab lives in the LDS the operand stages
// used, after the block barrier that ends the main loop.
#pragma once

#include "gemm_core.hpp"
#include "mr_common.hpp"

namespace mr {

constexpr int kSlabLd = 64 + 4;            // floats per slab row
constexpr int kSlabRows = 64;
constexpr int kSlabFloats = kSlabRows * kSlabLd;  // one wave's slab: 17 KB

// LDS writes by some lanes of a wave are read by other lanes of the same
// wave: wait for them, and keep the compiler from moving accesses across.
__device__ __forceinline__ void slab_fence() {
  // s_waitcnt lgkmcnt(0): vmcnt [3:0] and [15:14] and expcnt [6:4] at their
  // maxima, lgkmcnt [11:8] = 0
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Rows 32 h .. 32 h + 31 of the slab = the 32 rows of blocks (a0 | a1),
// columns 0..63.
__device__ __forceinline__ void slab_put(float* slab, int h, const v16f& a0, const v16f& a1, int lane) {
  const int c = lane & 31;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 32 * h + f32_row(lane, v);
    slab[r * kSlabLd + c] = a0[v];
    slab[r * kSlabLd + 32 + c] = a1[v];
  }
}

// f(r, c, v[8]) for the 512 row chunks (row r, columns c .. c+7), eight per
// lane; when f returns true, v is written back into the slab.
template <typename F>
__device__ __forceinline__ void slab_rows(float* slab, int lane, F&& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lane + 64 * i;
    const int r = q >> 3, c = (q & 7) * 8;
    float* p = slab + r * kSlabLd + c;
    const v4f x0 = *reinterpret_cast<const v4f*>(p);
    const v4f x1 = *reinterpret_cast<const v4f*>(p + 4);
    float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    if (f(r, c, v)) {
      *reinterpret_cast<v4f*>(p) = v4f{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<v4f*>(p + 4) = v4f{v[4], v[5], v[6], v[7]};
    }
  }
}

// f(c, r, v[8]) for the 512 column chunks (column c, rows r .. r+7), eight
// per lane; eight consecutive lanes cover the 64 rows of one column.
template <typename F>
__device__ __forceinline__ void slab_cols(const float* slab, int lane, F&& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = lane + 64 * i;
    const int c = q >> 3, r = (q & 7) * 8;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = slab[(r + e) * kSlabLd + c];
    f(c, r, v);
  }
}

// Split 8 floats into hi / lo fp16 vectors (split_f32 elementwise).
__device__ __forceinline__ void split8(const float (&v)[8], v8h& hi, v8h& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 h, l;
    split_f32(v[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// A whole tile of a GEMM whose waves form a grid WN wide, each wave owning
// RB x CB blocks of 32 x 32 (rows wm * 32 RB .., columns wn * 32 CB ..; RB
// and CB even), stored by 64 x 64 slabs:
//   out[r][c] = alpha acc + beta cin[r][c] (+ gamma on the diagonal)
// (cin optional: cin_hi == NULL) stored in split form at out (row stride
// ldo) and, transposed, at t (row stride ldt: t[c][r] = out[r][c]); cin has
// out's layout.  out_lo or t_lo NULL: that lo half is not stored (outputs
// only ever read as fp16 operands).  E is the type the combination is formed in before the
// float32 rounding.  diag: a symmetric output's diagonal tile (m0 == n0,
// t == out): only elements with r <= c are stored, and the mirror stores
// only those with r < c, so the tile's lower triangle is the mirror of its
// upper one (16-byte stores away from the diagonal, 2-byte stores on the
// chunks it crosses).  The caller has passed a block barrier since the LDS
// was last used for operands; `lds` holds kSlabFloats floats per wave.
template <int RB, int WN, typename E, int CB = 2>
__device__ __forceinline__ void wide_store_tile(const v16f (&acc)[RB][CB], float* lds, int m0, int n0,
                                                _Float16* out_hi, _Float16* out_lo, int64_t ldo, _Float16* t_hi,
                                                _Float16* t_lo, int64_t ldt, const _Float16* cin_hi,
                                                const _Float16* cin_lo, E alpha, E beta, E gamma = E(0),
                                                bool diag = false) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  static_assert(RB % 2 == 0 && CB % 2 == 0, "64 x 64 slabs");
  float* slab = lds + wave * kSlabFloats;
  // one 64 x 64 slab per call, block indices known at compile time (a
  // runtime index into acc would put the accumulators in scratch memory)
  auto one_slab = [&](auto sl_c) __attribute__((always_inline)) {
    constexpr int sl = decltype(sl_c)::value;
    constexpr int rb = 2 * (sl / (CB / 2)), cb = 2 * (sl % (CB / 2));
    slab_put(slab, 0, acc[rb][cb], acc[rb][cb + 1], lane);
    slab_put(slab, 1, acc[rb + 1][cb], acc[rb + 1][cb + 1], lane);
    slab_fence();
    const int r0 = m0 + wm * 32 * RB + rb * 32, c0 = n0 + wn * 32 * CB + cb * 32;
    slab_rows(slab, lane, [&](int r, int c, float (&v)[8]) {
      const int gr = r0 + r, gc = c0 + c;
      if (diag && gr > gc + 7) return false;  // wholly below the diagonal
      const int64_t idx = (int64_t)gr * ldo + gc;
      v8h ch = {}, cl = {};
      if (cin_hi) {
        ch = *reinterpret_cast<const v8h*>(cin_hi + idx);
        cl = *reinterpret_cast<const v8h*>(cin_lo + idx);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        E val = alpha * (E)v[e];
        if (cin_hi) val += beta * (E)join_f32(ch[e], cl[e]);
        if (diag && gr == gc + e) val += gamma;
        v[e] = (float)val;
      }
      v8h hh, ll;
      split8(v, hh, ll);
      if (!diag || gr <= gc) {
        *reinterpret_cast<v8h*>(out_hi + idx) = hh;
        if (out_lo) *reinterpret_cast<v8h*>(out_lo + idx) = ll;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gc + e >= gr) {
            out_hi[idx + e] = hh[e];
            if (out_lo) out_lo[idx + e] = ll[e];
          }
      }
      return true;
    });
    slab_fence();
    slab_cols(slab, lane, [&](int c, int r, const float (&v)[8]) {
      const int gc = c0 + c, gr = r0 + r;  // source rows gr .. gr+7 of column gc
      if (diag && gr >= gc) return;        // no source element above the diagonal
      const int64_t tidx = (int64_t)gc * ldt + gr;
      v8h hh, ll;
      split8(v, hh, ll);
      if (!diag || gr + 7 < gc) {
        *reinterpret_cast<v8h*>(t_hi + tidx) = hh;
        if (t_lo) *reinterpret_cast<v8h*>(t_lo + tidx) = ll;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gr + e < gc) {
            t_hi[tidx + e] = hh[e];
            if (t_lo) t_lo[tidx + e] = ll[e];
          }
      }
    });
    slab_fence();
  };
  static_for<RB * CB / 4>(one_slab);
}

}  // namespace mr
