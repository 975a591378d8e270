// MFMA tile cores for gfx950.
//
// Every core computes a block tile of C = A * B^T where row i of A and row j
// of B are indexed along the contraction k.  With symmetric operands (every
// product of the coupled Newton iteration, the Gram of G's rows) this "NT"
// form reads both operands along contiguous rows; the Gram cores can also read
// an operand "transposed" (element (i, k) at ptr[k * ld + i]), which the right
// Gram G^T G needs, and take float32 inputs widened to float64 (float32
// products are exact in float64).
//
// Cores (float32, float64 and split-fp16 arithmetic):
//   f32_nt_tile, f64_tile, x3_nt_tile   128 x 128, register-staged loads
//   f64dl_nt_tile, f64g_tile, x3dl_nt_tile   128 x 128, direct-to-LDS copies
//   x3w_nt_tile   256 x 256, direct-to-LDS copies, one accumulator
// The 128 x 128 cores run 256 threads = 4 waves in a 2 x 2 grid, each wave
// owning a 64 x 64 sub-tile; x3w_nt_tile runs 8 waves in a 2 x 4 grid of
// 128 x 64.  A and B chunks are staged through LDS stages.  Within a k-chunk
// each lane reads a run of consecutive k for its row with 128-bit LDS reads;
// consecutive MFMAs consume that run element by element.  The k order inside
// a chunk is therefore permuted, identically for A and B, which leaves the
// sum unchanged.
#pragma once

#include "mr_common.hpp"

namespace mr {

// ------------------------------------------------------------------ float32

struct F32Tile {
  static constexpr int BM = 128, BN = 128, BK = 32, PAD = 4, LDW = BK + PAD;
  static constexpr int THREADS = 256;
  static constexpr int STAGE = (BM + BN) * LDW;         // floats per LDS stage (A then B)
  static constexpr int LDS_FLOATS = 2 * STAGE;  // two stages
};

// Load a BM x BK chunk (rows r0.., k0..) of a K-contiguous float32 operand
// into registers.  VEC=4 needs ld % 4 == 0, K % 4 == 0 and a 16-byte aligned
// base; VEC=1 has element guards.
template <int VEC>
struct F32Loader {
  static constexpr int BK = F32Tile::BK;
  static constexpr int PER = (F32Tile::BM * BK) / (F32Tile::THREADS * VEC);
  static constexpr int VPR = BK / 4;  // float4 per row
  v4f reg[VEC == 4 ? PER : 1];
  float sreg[VEC == 1 ? PER : 1];

  __device__ __forceinline__ void load(const float* __restrict__ P, int64_t ld, int rows, int K, int r0,
                                       int k0, int tid) {
    if constexpr (VEC == 4) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = tid + p * F32Tile::THREADS;
        const int row = idx / VPR;
        const int kq = (idx % VPR) * 4;
        const int gr = r0 + row, gk = k0 + kq;
        v4f v = {0.f, 0.f, 0.f, 0.f};
        if (gr < rows && gk < K) v = *reinterpret_cast<const v4f*>(P + (int64_t)gr * ld + gk);
        reg[p] = v;
      }
    } else {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = tid + p * F32Tile::THREADS;
        const int row = idx / BK;
        const int kk = idx % BK;
        const int gr = r0 + row, gk = k0 + kk;
        sreg[p] = (gr < rows && gk < K) ? P[(int64_t)gr * ld + gk] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(float* __restrict__ s, int tid) const {
    if constexpr (VEC == 4) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = tid + p * F32Tile::THREADS;
        *reinterpret_cast<v4f*>(s + (idx / VPR) * F32Tile::LDW + (idx % VPR) * 4) = reg[p];
      }
    } else {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = tid + p * F32Tile::THREADS;
        s[(idx / BK) * F32Tile::LDW + (idx % BK)] = sreg[p];
      }
    }
  }
};

__device__ __forceinline__ void f32_chunk(const float* __restrict__ sA, const float* __restrict__ sB,
                                          v16f (&acc)[2][2], int lane, int wm, int wn) {
  const int koff = (lane >> 5) * 8;
#pragma unroll
  for (int g = 0; g < F32Tile::BK / 16; ++g) {
    v4f a[2][2], b[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float* pa = sA + (wm * 64 + rb * 32 + (lane & 31)) * F32Tile::LDW + g * 16 + koff;
      a[rb][0] = *reinterpret_cast<const v4f*>(pa);
      a[rb][1] = *reinterpret_cast<const v4f*>(pa + 4);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float* pb = sB + (wn * 64 + cb * 32 + (lane & 31)) * F32Tile::LDW + g * 16 + koff;
      b[cb][0] = *reinterpret_cast<const v4f*>(pb);
      b[cb][1] = *reinterpret_cast<const v4f*>(pb + 4);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = mfma_f32_32x32x2(a[rb][i >> 2][i & 3], b[cb][i >> 2][i & 3], acc[rb][cb]);
  }
}

// acc[rb][cb] holds the 32 x 32 MFMA block (rb, cb) of this wave's 64 x 64
// sub-tile.  lds: F32Tile::LDS_FLOATS floats.  With DBUF the next k-chunk is
// written to the other LDS stage while the current one is consumed, so each
// chunk costs one barrier.
template <int VEC>
__device__ __forceinline__ void f32_nt_tile(const float* __restrict__ A, int64_t lda,
                                            const float* __restrict__ B, int64_t ldb, int M, int N,
                                            int K, int m0, int n0, float* __restrict__ lds,
                                            v16f (&acc)[2][2]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BK = F32Tile::BK;
  constexpr int AOFF = 0, BOFF = F32Tile::BM * F32Tile::LDW;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;

  F32Loader<VEC> la, lb;
  la.load(A, lda, M, K, m0, 0, tid);
  lb.load(B, ldb, N, K, n0, 0, tid);
  la.store(lds + AOFF, tid);
  lb.store(lds + BOFF, tid);
  __syncthreads();
  int stage = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) {
      la.load(A, lda, M, K, m0, k0 + BK, tid);
      lb.load(B, ldb, N, K, n0, k0 + BK, tid);
    }
    const float* cur = lds + stage * F32Tile::STAGE;
    f32_chunk(cur + AOFF, cur + BOFF, acc, lane, wm, wn);
    if (more) {
      float* nxt = lds + (stage ^ 1) * F32Tile::STAGE;
      la.store(nxt + AOFF, tid);
      lb.store(nxt + BOFF, tid);
    }
    __syncthreads();
    stage ^= 1;
  }
  
}

// ------------------------------------------------------------- split fp16
// C = A * B^T for float32-accurate operands on the fp16 matrix cores.  Every
// operand is stored split: x = hi + 2^-11 lo with hi = fp16(x) and
// lo = fp16((x - hi) * 2^11) (x - hi is exact in float32), as two fp16 arrays
// of the operand's shape (the producers write this form, so the GEMM loop only
// copies fp16 tiles).  Then
//   C = sum hi_a hi_b + 2^-11 * sum (hi_a lo_b + lo_a hi_b),
// the two sums in separate float32 accumulators.  Products of 11-bit
// significands are exact in float32; the dropped lo*lo term and the rounding
// of lo leave about 2^-22 relative error per product (float32: 2^-24), and
// the float32 accumulation is the same as on the float32 matrix cores.
struct X3Tile {
  static constexpr int BM = 128, BN = 128, BK = 32, PAD = 8, LDW = BK + PAD;  // halves per LDS row
  static constexpr int THREADS = 256;
  static constexpr int ARR = BM * LDW;  // halves per array (A_hi, A_lo, B_hi, B_lo)
  static constexpr int STAGE = 4 * ARR;
  static constexpr int LDS_HALVES = 2 * STAGE;  // two stages
};

struct SplitRef {
  const _Float16* hi;
  const _Float16* lo;
};

__device__ __forceinline__ void split_f32(float x, _Float16& h, _Float16& l) {
  h = (_Float16)x;
  l = (_Float16)((x - (float)h) * 2048.0f);
}
__device__ __forceinline__ float join_f32(_Float16 h, _Float16 l) { return (float)h + (float)l * (1.0f / 2048.0f); }

// Loads a BM x BK chunk of a K-contiguous split operand.  VEC = 8 (16-byte
// loads; needs ld and K multiples of 8 and 16-byte aligned arrays) or 1.
template <int VEC>
struct SplitLoader {
  static constexpr int BK = X3Tile::BK;
  static constexpr int PER = (X3Tile::BM * BK) / (X3Tile::THREADS * 8);  // groups of 8 halves
  static constexpr int GPR = BK / 8;
  v8h rh[PER], rl[PER];

  __device__ __forceinline__ void load(SplitRef P, int64_t ld, int rows, int K, int r0, int k0, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int row, grp;
      tile_slot<GPR>(tid + p * X3Tile::THREADS, row, grp);
      const int gr = r0 + row, gk = k0 + grp * 8;
      const int64_t off = (int64_t)gr * ld + gk;
      if constexpr (VEC == 8) {
        v8h h = {}, l = {};
        if (gr < rows && gk < K) {
          h = *reinterpret_cast<const v8h*>(P.hi + off);
          l = *reinterpret_cast<const v8h*>(P.lo + off);
        }
        rh[p] = h;
        rl[p] = l;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = gr < rows && gk + e < K;
          rh[p][e] = ok ? P.hi[off + e] : (_Float16)0.0f;
          rl[p][e] = ok ? P.lo[off + e] : (_Float16)0.0f;
        }
      }
    }
  }
  __device__ __forceinline__ void store(_Float16* __restrict__ hi, _Float16* __restrict__ lo, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int row, grp;
      tile_slot<GPR>(tid + p * X3Tile::THREADS, row, grp);
      const int off = row * X3Tile::LDW + grp * 8;
      *reinterpret_cast<v8h*>(hi + off) = rh[p];
      *reinterpret_cast<v8h*>(lo + off) = rl[p];
    }
  }
};

__device__ __forceinline__ void x3_chunk(const _Float16* __restrict__ st, v16f (&acc)[2][2], v16f (&acc2)[2][2],
                                         int lane, int wm, int wn) {
  const _Float16* Ahi = st;
  const _Float16* Alo = st + X3Tile::ARR;
  const _Float16* Bhi = st + 2 * X3Tile::ARR;
  const _Float16* Blo = st + 3 * X3Tile::ARR;
  const int koff = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < X3Tile::BK / 16; ++ks) {
    v8h ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int o = (wm * 64 + rb * 32 + (lane & 31)) * X3Tile::LDW + ks * 16 + koff;
      ah[rb] = *reinterpret_cast<const v8h*>(Ahi + o);
      al[rb] = *reinterpret_cast<const v8h*>(Alo + o);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int o = (wn * 64 + cb * 32 + (lane & 31)) * X3Tile::LDW + ks * 16 + koff;
      bh[cb] = *reinterpret_cast<const v8h*>(Bhi + o);
      bl[cb] = *reinterpret_cast<const v8h*>(Blo + o);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        acc[rb][cb] = mfma_f16_32x32x16(ah[rb], bh[cb], acc[rb][cb]);
        acc2[rb][cb] = mfma_f16_32x32x16(ah[rb], bl[cb], acc2[rb][cb]);
        acc2[rb][cb] = mfma_f16_32x32x16(al[rb], bh[cb], acc2[rb][cb]);
      }
  }
}

// Result in acc (combined: acc + 2^-11 acc2).
template <int VEC>
__device__ __forceinline__ void x3_nt_tile(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int K,
                                           int m0, int n0, _Float16* __restrict__ lds, v16f (&acc)[2][2]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BK = X3Tile::BK;
  v16f acc2[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[rb][cb][v] = 0.f;
        acc2[rb][cb][v] = 0.f;
      }
  SplitLoader<VEC> la, lb;
  la.load(A, lda, M, K, m0, 0, tid);
  lb.load(B, ldb, N, K, n0, 0, tid);
  la.store(lds, lds + X3Tile::ARR, tid);
  lb.store(lds + 2 * X3Tile::ARR, lds + 3 * X3Tile::ARR, tid);
  __syncthreads();
  int stage = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) {
      la.load(A, lda, M, K, m0, k0 + BK, tid);
      lb.load(B, ldb, N, K, n0, k0 + BK, tid);
    }
    x3_chunk(lds + stage * X3Tile::STAGE, acc, acc2, lane, wm, wn);
    if (more) {
      _Float16* nxt = lds + (stage ^ 1) * X3Tile::STAGE;
      la.store(nxt, nxt + X3Tile::ARR, tid);
      lb.store(nxt + 2 * X3Tile::ARR, nxt + 3 * X3Tile::ARR, tid);
    }
    __syncthreads();
    stage ^= 1;
  }
  
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = acc[rb][cb][v] + acc2[rb][cb][v] * (1.0f / 2048.0f);
}

// The same product and accumulator layout with the operand chunks copied
// straight from global memory into LDS (direct-to-LDS copies, no staging
// registers and no LDS store instructions), chunks of 32 along k in two
// stages: a wave waits for its own copies of the next chunk and a bare
// s_barrier publishes them, so the copies of the chunk after stay in flight
// during the MFMAs.  Stage layout: A_hi, A_lo, B_hi, B_lo, each 128 rows of
// four 16-byte units in the dl_slot order.  Preconditions (checked by the
// caller): K a multiple of 32, lda and ldb multiples of 8, 16-byte aligned
// arrays.  Rows beyond M or N are read from row M - 1 or N - 1: they only feed
// outputs that are never stored.
struct X3DL {
  static constexpr int BK = 32, UPR = BK / 8;
  static constexpr int AU = X3Tile::BM * UPR;  // 16-byte units per array and stage
  static constexpr int STAGE_BYTES = 4 * AU * 16;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int CPA = AU / X3Tile::THREADS;  // copies per lane and array
  static_assert(CPA * X3Tile::THREADS == AU, "copies cover the chunk");
};

__device__ __forceinline__ void x3dl_issue(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int m0,
                                           int n0, int k0, unsigned char* stage, int wave, int lane) {
#pragma unroll
  for (int arr = 0; arr < 4; ++arr) {
    const bool isA = arr < 2;
    const int64_t ld = isA ? lda : ldb;
    const int r0 = isA ? m0 : n0, rlast = (isA ? M : N) - 1 - r0;
    // scalar base (row r0, column k0) plus a 32-bit lane byte offset within
    // the tile's rows: one copy instruction each
    const char* P = wave_uniform((arr == 0 ? A.hi : arr == 1 ? A.lo : arr == 2 ? B.hi : B.lo) + (int64_t)r0 * ld + k0);
#pragma unroll
    for (int j = 0; j < X3DL::CPA; ++j) {
      const int base_u = (j * (X3Tile::THREADS / 64) + wave) * 64;
      const int u = base_u + lane;
      const int row = u / X3DL::UPR;
      const int kg = dl_slot(row, u % X3DL::UPR, X3DL::UPR);  // the map is its own inverse
      uint32_t off = ((uint32_t)min(row, rlast) * (uint32_t)ld + (uint32_t)(kg * 8)) * 2u;
      asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
      __builtin_amdgcn_global_load_lds((global_void_ptr)(P + off),
                                       (lds_void_ptr)(stage + (arr * X3DL::AU + base_u) * 16), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void x3dl_chunk(const unsigned char* __restrict__ st, v16f (&acc)[2][2],
                                           v16f (&acc2)[2][2], int lane, int wm, int wn) {
  constexpr int AB = X3DL::AU * 16;  // bytes per array
#pragma unroll
  for (int ks = 0; ks < X3DL::BK / 16; ++ks) {
    const int kg = ks * 2 + (lane >> 5);
    v8h ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = wm * 64 + rb * 32 + (lane & 31);
      const int o = (r * X3DL::UPR + dl_slot(r, kg, X3DL::UPR)) * 16;
      ah[rb] = *reinterpret_cast<const v8h*>(st + o);
      al[rb] = *reinterpret_cast<const v8h*>(st + AB + o);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = wn * 64 + cb * 32 + (lane & 31);
      const int o = (r * X3DL::UPR + dl_slot(r, kg, X3DL::UPR)) * 16;
      bh[cb] = *reinterpret_cast<const v8h*>(st + 2 * AB + o);
      bl[cb] = *reinterpret_cast<const v8h*>(st + 3 * AB + o);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        acc[rb][cb] = mfma_f16_32x32x16(ah[rb], bh[cb], acc[rb][cb]);
        acc2[rb][cb] = mfma_f16_32x32x16(ah[rb], bl[cb], acc2[rb][cb]);
        acc2[rb][cb] = mfma_f16_32x32x16(al[rb], bh[cb], acc2[rb][cb]);
      }
  }
}

struct X3DLFrag {
  v8h ah[2], al[2], bh[2], bl[2];
};

__device__ __forceinline__ void x3dl_read(const unsigned char* __restrict__ st, int ks, X3DLFrag& f, int lane, int wm,
                                          int wn) {
  constexpr int AB = X3DL::AU * 16;  // bytes per array
  const int kg = ks * 2 + (lane >> 5);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = wm * 64 + rb * 32 + (lane & 31);
    const int o = (r * X3DL::UPR + dl_slot(r, kg, X3DL::UPR)) * 16;
    f.ah[rb] = *reinterpret_cast<const v8h*>(st + o);
    f.al[rb] = *reinterpret_cast<const v8h*>(st + AB + o);
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = wn * 64 + cb * 32 + (lane & 31);
    const int o = (r * X3DL::UPR + dl_slot(r, kg, X3DL::UPR)) * 16;
    f.bh[cb] = *reinterpret_cast<const v8h*>(st + 2 * AB + o);
    f.bl[cb] = *reinterpret_cast<const v8h*>(st + 3 * AB + o);
  }
}

__device__ __forceinline__ void x3dl_mfma(const X3DLFrag& f, v16f (&acc)[2][2], v16f (&acc2)[2][2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      acc[rb][cb] = mfma_f16_32x32x16(f.ah[rb], f.bh[cb], acc[rb][cb]);
      acc2[rb][cb] = mfma_f16_32x32x16(f.ah[rb], f.bl[cb], acc2[rb][cb]);
      acc2[rb][cb] = mfma_f16_32x32x16(f.al[rb], f.bh[cb], acc2[rb][cb]);
    }
}

// 8 reads spread over 12 products (the scheme of x3w_sched_overlap)
__device__ __forceinline__ void x3dl_sched_overlap() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}


__device__ __forceinline__ void x3dl_nt_tile(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int K,
                                             int m0, int n0, unsigned char* __restrict__ lds, v16f (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
  const int wm = wave >> 1, wn = wave & 1;
  v16f acc2[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[rb][cb][v] = 0.f;
        acc2[rb][cb][v] = 0.f;
      }
  const int nch = K / X3DL::BK;
  // fragment reads one k-step ahead, across chunk boundaries too (the scheme
  // of x3w_nt_tile)
  static_assert(X3DL::BK == 32, "two k-steps per chunk");
  X3DLFrag f0, f1;
  if (nch > 0) {
    x3dl_issue(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nch > 1) x3dl_issue(A, lda, B, ldb, M, N, m0, n0, X3DL::BK, lds + X3DL::STAGE_BYTES, wave, lane);
    x3dl_read(lds, 0, f0, lane, wm, wn);
  }
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = c + s;
      if (cc < nch) {
        unsigned char* st = lds + s * X3DL::STAGE_BYTES;
        x3dl_read(st, 1, f1, lane, wm, wn);
        x3dl_mfma(f0, acc, acc2);
        x3dl_sched_overlap();
        wait_lgkmcnt0();
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // stage s is free, chunk cc + 1 is in stage s ^ 1
        asm volatile("" ::: "memory");
        if (cc + 2 < nch) x3dl_issue(A, lda, B, ldb, M, N, m0, n0, (cc + 2) * X3DL::BK, st, wave, lane);
        // (after the last chunk this reads a stale stage; those fragments are never used)
        x3dl_read(lds + (s ^ 1) * X3DL::STAGE_BYTES, 0, f0, lane, wm, wn);
        x3dl_mfma(f1, acc, acc2);
        x3dl_sched_overlap();
      }
    }
  }
  __syncthreads();  // no wave leaves (or reuses the LDS) while another may still read the last stage
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = acc[rb][cb][v] + acc2[rb][cb][v] * (1.0f / 2048.0f);
}

// Direct-to-LDS core where its preconditions hold (VEC 8: 16-byte aligned
// operands, leading dimensions multiples of 8), else the register-staged one.
template <int VEC>
__device__ __forceinline__ void x3_nt_tile_auto(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int K,
                                                int m0, int n0, unsigned char* __restrict__ lds, v16f (&acc)[2][2]) {
  static_assert(X3DL::LDS_BYTES <= 2 * X3Tile::LDS_HALVES, "both cores fit the same LDS");
  if (VEC == 8 && K % X3DL::BK == 0)
    x3dl_nt_tile(A, lda, B, ldb, M, N, K, m0, n0, lds, acc);
  else
    x3_nt_tile<VEC>(A, lda, B, ldb, M, N, K, m0, n0, reinterpret_cast<_Float16*>(lds), acc);
}

// Wide split-fp16 tile for operands whose B side is bounded: 256 x 256 block
// tile, eight waves in a 2 x 4 grid (128 x 64 each: 4 x 2 blocks of 32 x 32),
// direct-to-LDS copies in 32-deep chunks, two stages (128 KB).  One float32
// accumulator takes all three products: with B's hi half multiplied by 2^11
// in registers (exact: a power of two, and |B| < 32 keeps 2^11 hi_b inside
// fp16's range),
//   2^11 hi_a hi_b + hi_a lo_b + lo_a hi_b = 2^11 (hi_a hi_b + 2^-11 (hi_a lo_b + lo_a hi_b)),
// whose float32 sum rounds like the larger of the two separate sums of
// x3_nt_tile (the hi_a hi_b sum sets the rounding in both), so both forms
// carry the same accuracy; the single accumulator halves the accumulator
// registers, which is what lets one wave hold a 128 x 64 tile.
// Preconditions (checked by the caller): K a multiple of 32, lda and ldb
// multiples of 8, 16-byte aligned arrays, every |B| < 32.  Rows beyond M or N
// are read from row M - 1 or N - 1: they only feed outputs never stored.
template <int BK_, int NST_, int WN_>
struct X3WCfg {
  static constexpr int BM = 256, BN = 256, WM = 2, WN = WN_, THREADS = 64 * WM * WN;
  static constexpr int RB = BM / WM / 32, CB = BN / WN / 32;
  static constexpr int BK = BK_, NST = NST_, UPR = BK / 8;
  static constexpr int AU = BM * UPR;  // 16-byte units per array and stage (BM == BN)
  static constexpr int STAGE_BYTES = 4 * AU * 16;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int CPA = AU / THREADS;  // copies per lane and array
  static constexpr int LPC = 4 * CPA;       // copies per lane and chunk
  static_assert(BM == BN && CB % 2 == 0 && RB % 2 == 0 && CPA * THREADS == AU, "square tile, 64 x 64 wave slabs");
  static_assert(BK % 16 == 0 && 32 % BK == 0 && NST >= 2 && LDS_BYTES <= 160 * 1024, "chunk depth and stages");
};
using X3W = X3WCfg<32, 2, 4>;  // 32-deep chunks, two stages, 2 x 4 waves

__device__ __forceinline__ void x3w_issue(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int m0,
                                          int n0, int k0, unsigned char* stage, int wave, int lane) {
  // Copy j of a lane covers row lrow + j * THREADS / UPR of the tile, in the
  // same k-group for every j (the slot map repeats every 16 rows); rows past
  // the last are clamped to it.  Each copy is one instruction: a scalar base
  // (the array at row r0, column k0) plus a 32-bit lane byte offset within
  // the tile's rows (under 2 * 256 * ld bytes).
  static_assert((X3W::THREADS / 16) % X3W::UPR == 0, "one k-group per lane");
  const int lu = wave * 64 + lane;
  const int lrow = lu / X3W::UPR;
  const int kg = dl_slot(lrow, lu % X3W::UPR, X3W::UPR);  // the map is its own inverse
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const int64_t ld = side == 0 ? lda : ldb;
    const int r0 = side == 0 ? m0 : n0, rlast = (side == 0 ? M : N) - 1 - r0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int arr = side * 2 + half;
      const char* P =
          wave_uniform((arr == 0 ? A.hi : arr == 1 ? A.lo : arr == 2 ? B.hi : B.lo) + (int64_t)r0 * ld + k0);
#pragma unroll
      for (int j = 0; j < X3W::CPA; ++j) {
        const int base_u = (j * (X3W::THREADS / 64) + wave) * 64;
        const uint32_t row = (uint32_t)min(lrow + j * (X3W::THREADS / X3W::UPR), rlast);
        uint32_t off = (row * (uint32_t)ld + (uint32_t)(kg * 8)) * 2u;
        asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
        __builtin_amdgcn_global_load_lds((global_void_ptr)(P + off),
                                         (lds_void_ptr)(stage + (arr * X3W::AU + base_u) * 16), 16, 0, 0);
      }
    }
  }
}

// One k-step's operand fragments of a wave (hi and lo halves of its A rows
// and B columns), the reads that fill them and the products that use them.
struct X3WFrag {
  v8h ah[X3W::RB], al[X3W::RB], bh[X3W::CB], bl[X3W::CB];
};

__device__ __forceinline__ void x3w_read(const unsigned char* __restrict__ st, int ks, X3WFrag& f, int lane, int wm,
                                         int wn) {
  constexpr int AB = X3W::AU * 16;  // bytes per array
  const int kg = ks * 2 + (lane >> 5);
#pragma unroll
  for (int rb = 0; rb < X3W::RB; ++rb) {
    const int r = wm * (X3W::BM / X3W::WM) + rb * 32 + (lane & 31);
    const int o = (r * X3W::UPR + dl_slot(r, kg, X3W::UPR)) * 16;
    f.ah[rb] = *reinterpret_cast<const v8h*>(st + o);
    f.al[rb] = *reinterpret_cast<const v8h*>(st + AB + o);
  }
#pragma unroll
  for (int cb = 0; cb < X3W::CB; ++cb) {
    const int r = wn * (X3W::BN / X3W::WN) + cb * 32 + (lane & 31);
    const int o = (r * X3W::UPR + dl_slot(r, kg, X3W::UPR)) * 16;
    f.bh[cb] = *reinterpret_cast<const v8h*>(st + 2 * AB + o);
    f.bl[cb] = *reinterpret_cast<const v8h*>(st + 3 * AB + o);
  }
}

__device__ __forceinline__ void x3w_mfma(const X3WFrag& f, v16f (&acc)[X3W::RB][X3W::CB]) {
#pragma unroll
  for (int cb = 0; cb < X3W::CB; ++cb) {
#pragma unroll
    for (int rb = 0; rb < X3W::RB; ++rb) acc[rb][cb] = mfma_f16_32x32x16(f.al[rb], f.bh[cb], acc[rb][cb]);
    const v8h bs = f.bh[cb] * (_Float16)2048.0f;
#pragma unroll
    for (int rb = 0; rb < X3W::RB; ++rb) {
      acc[rb][cb] = mfma_f16_32x32x16(f.ah[rb], f.bl[cb], acc[rb][cb]);
      acc[rb][cb] = mfma_f16_32x32x16(f.ah[rb], bs, acc[rb][cb]);
    }
  }
}

// Instruction order for a region holding one k-step's products and the next
// k-step's fragment reads: the reads spread evenly over the products.
__device__ __forceinline__ void x3w_sched_overlap() {
  constexpr int NR = 2 * (X3W::RB + X3W::CB), NM = 3 * X3W::RB * X3W::CB;
  constexpr int PER = NM / NR;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // products
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR, 0);
}

// Result in acc: float32 sums of the wave's 4 x 2 blocks (layout of x3w_for_each).
__device__ __forceinline__ void x3w_nt_tile(SplitRef A, int64_t lda, SplitRef B, int64_t ldb, int M, int N, int K,
                                            int m0, int n0, unsigned char* __restrict__ lds,
                                            v16f (&acc)[X3W::RB][X3W::CB]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
  const int wm = wave / X3W::WN, wn = wave % X3W::WN;
#pragma unroll
  for (int rb = 0; rb < X3W::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < X3W::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;
  const int nch = K / X3W::BK;
  // Fragment reads one k-step ahead, across chunk boundaries too: a k-step's
  // products run while the next k-step's fragments are read, from the same
  // stage or, after the barrier, from the next one.  The barrier sits
  // between the two halves of a chunk's products: each wave has finished
  // reading the stage before it (LDS count 0) and holds the next chunk's
  // copies (vector-memory count 0).
  static_assert(X3W::NST == 2 && X3W::BK == 32, "two stages of two k-steps");
  X3WFrag f0, f1;
  if (nch > 0) {
    x3w_issue(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nch > 1) x3w_issue(A, lda, B, ldb, M, N, m0, n0, X3W::BK, lds + X3W::STAGE_BYTES, wave, lane);
    x3w_read(lds, 0, f0, lane, wm, wn);
  }
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = c + s;
      if (cc < nch) {
        unsigned char* st = lds + s * X3W::STAGE_BYTES;
        x3w_read(st, 1, f1, lane, wm, wn);
        x3w_mfma(f0, acc);
        x3w_sched_overlap();
        wait_lgkmcnt0();
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // stage s is free, chunk cc + 1 is in stage s ^ 1
        asm volatile("" ::: "memory");
        if (cc + 2 < nch) x3w_issue(A, lda, B, ldb, M, N, m0, n0, (cc + 2) * X3W::BK, st, wave, lane);
        // (after the last chunk this reads a stale stage; those fragments are never used)
        x3w_read(lds + (s ^ 1) * X3W::STAGE_BYTES, 0, f0, lane, wm, wn);
        x3w_mfma(f1, acc);
        x3w_sched_overlap();
      }
    }
  }
  __syncthreads();  // no wave leaves (or reuses the LDS) while another may still read the last stage
#pragma unroll
  for (int rb = 0; rb < X3W::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < X3W::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = acc[rb][cb][v] * (1.0f / 2048.0f);
}

template <typename F>
__device__ __forceinline__ void x3w_for_each(const v16f (&acc)[X3W::RB][X3W::CB], F&& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / X3W::WN, wn = wave % X3W::WN;
  static_for<X3W::RB * X3W::CB>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int rb = decltype(i_c)::value / X3W::CB, cb = decltype(i_c)::value % X3W::CB;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      f(wm * (X3W::BM / X3W::WM) + rb * 32 + f32_row(lane, v), wn * (X3W::BN / X3W::WN) + cb * 32 + (lane & 31),
        acc[rb][cb][v]);
  });
}

// Visit every accumulator element of the f32 core as (row, col) local to the
// block tile.
template <typename F>
__device__ __forceinline__ void f32_for_each(const v16f (&acc)[2][2], F&& f) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        f(wm * 64 + rb * 32 + f32_row(lane, v), wn * 64 + cb * 32 + (lane & 31), acc[rb][cb][v]);
}

// ------------------------------------------------------------------ float64

struct F64Tile {
  static constexpr int BM = 128, BN = 128, BK = 16, PAD = 2, LDW = BK + PAD;
  static constexpr int THREADS = 256;
  static constexpr int STAGE = (BM + BN) * LDW;  // doubles per LDS stage (A then B)
  static constexpr int LDS_DOUBLES = 2 * STAGE;  // two stages
};

// Loader of a BM x BK chunk of operand element (i, k), i in [r0, r0+BM),
// k in [k0, k0+BK), widened to double.
//   TRANS = false: element at P[i * ld + k]; TRANS = true: at P[k * ld + i].
//   VEC: elements per global load (4 for float, 2 for double; 1 = guarded scalar).
template <typename TIn, bool TRANS, int VEC>
struct F64Loader {
  static constexpr int BK = F64Tile::BK;
  static constexpr int ELEMS = F64Tile::BM * BK;
  static constexpr int PER = ELEMS / (F64Tile::THREADS * VEC);
  static constexpr int VPR_K = BK / VEC;            // vectors per row when !TRANS
  double reg[PER * VEC];

  // TRANS (VEC consecutive i of one k per load): consecutive lanes take
  // consecutive k, so the transposed LDS stores of a wave land on
  // consecutive doubles of a row (16 lanes per row) instead of rows VEC
  // apart, which put eight lanes on one bank pair; the global loads then
  // cover 4 VEC floats of 16 rows per wave instruction.
  __device__ __forceinline__ static void trans_slot(int idx, int& i, int& k) {
    k = idx % BK;
    i = (idx / BK) * VEC;
  }

  __device__ __forceinline__ void load(const TIn* __restrict__ P, int64_t ld, int rows, int K, int r0,
                                       int k0, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + p * F64Tile::THREADS;
      int i, k;
      if constexpr (!TRANS && VEC == 2 && F64Tile::PAD == 2) {
        // 16-byte groups, 8 per 144-byte row: the conflict-free store order
        tile_slot<VPR_K>(idx, i, k);
        k *= VEC;
      } else if constexpr (!TRANS) {
        i = idx / VPR_K;
        k = (idx % VPR_K) * VEC;
      } else if constexpr (VEC == 1) {  // the element path's own order (store())
        k = idx / F64Tile::BM;
        i = idx % F64Tile::BM;
      } else {
        trans_slot(idx, i, k);
      }
      const int gi = r0 + i, gk = k0 + k;
      if constexpr (VEC == 1) {
        reg[p] = (gi < rows && gk < K) ? (double)P[TRANS ? (int64_t)gk * ld + gi : (int64_t)gi * ld + gk]
                                       : 0.0;
      } else {
        // VEC consecutive elements along the contiguous index; the host only
        // picks VEC > 1 when that index's extent is a multiple of VEC, so the
        // vector is all-in or all-out.
        const bool ok = gi < rows && gk < K;
        const int64_t off = TRANS ? (int64_t)gk * ld + gi : (int64_t)gi * ld + gk;
        if constexpr (sizeof(TIn) == 4) {
          v4f v = {0.f, 0.f, 0.f, 0.f};
          if (ok) v = *reinterpret_cast<const v4f*>(P + off);
#pragma unroll
          for (int e = 0; e < 4; ++e) reg[p * 4 + e] = (double)v[e];
        } else {
          v2d v = {0.0, 0.0};
          if (ok) v = *reinterpret_cast<const v2d*>(P + off);
          reg[p * 2 + 0] = v[0];
          reg[p * 2 + 1] = v[1];
        }
      }
    }
  }
  __device__ __forceinline__ void store(double* __restrict__ s, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = tid + p * F64Tile::THREADS;
      if constexpr (VEC == 1) {
        int i, k;
        if constexpr (!TRANS) {
          i = idx / BK;
          k = idx % BK;
        } else {
          k = idx / F64Tile::BM;
          i = idx % F64Tile::BM;
        }
        s[i * F64Tile::LDW + k] = reg[p];
      } else if constexpr (!TRANS) {
        int i, k;
        if constexpr (VEC == 2 && F64Tile::PAD == 2) {
          tile_slot<VPR_K>(idx, i, k);
          k *= VEC;
        } else {
          i = idx / VPR_K;
          k = (idx % VPR_K) * VEC;
        }
#pragma unroll
        for (int e = 0; e < VEC; e += 2) {
          v2d v = {reg[p * VEC + e], reg[p * VEC + e + 1]};
          *reinterpret_cast<v2d*>(s + i * F64Tile::LDW + k + e) = v;
        }
      } else {
        int i, k;
        trans_slot(idx, i, k);
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[(i + e) * F64Tile::LDW + k] = reg[p * VEC + e];
      }
    }
  }
};

// Fragments are read two k-steps at a time (one 128-bit LDS read per operand
// block) to keep register pressure low enough for two waves per SIMD.
__device__ __forceinline__ void f64_chunk(const double* __restrict__ sA, const double* __restrict__ sB,
                                          v4d (&acc)[4][4], int lane, int wm, int wn) {
  const int koff = (lane >> 4) * 4;
  const double* pa0 = sA + (wm * 64 + (lane & 15)) * F64Tile::LDW + koff;
  const double* pb0 = sB + (wn * 64 + (lane & 15)) * F64Tile::LDW + koff;
#pragma unroll
  for (int g = 0; g < F64Tile::BK / 16; ++g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v2d a[4], b[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        a[rb] = *reinterpret_cast<const v2d*>(pa0 + rb * 16 * F64Tile::LDW + g * 16 + 2 * h);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        b[cb] = *reinterpret_cast<const v2d*>(pb0 + cb * 16 * F64Tile::LDW + g * 16 + 2 * h);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma_f64_16x16x4(a[rb][i], b[cb][i], acc[rb][cb]);
    }
  }
}

// acc[rb][cb]: 16 x 16 MFMA block (rb, cb) of this wave's 64 x 64 sub-tile.
// lds: F64Tile::LDS_DOUBLES doubles.
template <typename TA, bool TRANSA, int VECA, typename TB, bool TRANSB, int VECB>
__device__ __forceinline__ void f64_tile(const TA* __restrict__ A, int64_t lda, const TB* __restrict__ B,
                                         int64_t ldb, int M, int N, int K, int m0, int n0,
                                         double* __restrict__ lds, v4d (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BK = F64Tile::BK;
  constexpr int AOFF = 0, BOFF = F64Tile::BM * F64Tile::LDW;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rb][cb][v] = 0.0;

  F64Loader<TA, TRANSA, VECA> la;
  F64Loader<TB, TRANSB, VECB> lb;
  la.load(A, lda, M, K, m0, 0, tid);
  lb.load(B, ldb, N, K, n0, 0, tid);
  la.store(lds + AOFF, tid);
  lb.store(lds + BOFF, tid);
  __syncthreads();
  int stage = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) {
      la.load(A, lda, M, K, m0, k0 + BK, tid);
      lb.load(B, ldb, N, K, n0, k0 + BK, tid);
    }
    const double* cur = lds + stage * F64Tile::STAGE;
    f64_chunk(cur + AOFF, cur + BOFF, acc, lane, wm, wn);
    if (more) {
      double* nxt = lds + (stage ^ 1) * F64Tile::STAGE;
      la.store(nxt + AOFF, tid);
      lb.store(nxt + BOFF, tid);
    }
    __syncthreads();
    stage ^= 1;
  }
  
}

// The same product (float64 operands along contiguous rows, NT) with the
// operand chunks copied straight from global memory into LDS: rows of BK = 16
// doubles as eight 16-byte units in the dl_slot order, two stages (64 KB).
// A lane reads the unit holding k = 4 (lane / 16) + 2h + {0, 1} of its row,
// the k order of f64_chunk, so both cores sum in the same order and agree
// bitwise.  Preconditions (checked by the caller): K a multiple of 16, lda
// and ldb even, 16-byte aligned arrays.  Rows beyond M or N are read from row
// M - 1 or N - 1: they only feed outputs that are never stored.  Symmetric
// outputs only: in a diagonal tile (m0 == n0) the blocks wholly below the
// diagonal are left at zero (f64_block_mode).
struct F64DL {
  static constexpr int BK = F64Tile::BK, UPR = BK / 2;
  static constexpr int AU = F64Tile::BM * UPR;  // 16-byte units per operand and stage
  static constexpr int STAGE_BYTES = 2 * AU * 16;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int CPO = AU / F64Tile::THREADS;  // copies per lane and operand
  static_assert(BK == 16 && CPO * F64Tile::THREADS == AU, "eight units per row, copies cover the chunk");
};

__device__ __forceinline__ void f64dl_issue(const double* __restrict__ A, int64_t lda, const double* __restrict__ B,
                                            int64_t ldb, int M, int N, int m0, int n0, int k0, unsigned char* stage,
                                            int wave, int lane) {
  // Copy j of a lane covers row lrow + j * THREADS / UPR of the tile, in the
  // same k-group for every j, rows past the last clamped to it.  Each copy is
  // one instruction: a scalar base (row r0, column k0) plus a 32-bit lane byte
  // offset within the tile's rows.
  static_assert((F64Tile::THREADS / 16) % F64DL::UPR == 0, "one k-group per lane");
  const int lu = wave * 64 + lane;
  const int lrow = lu / F64DL::UPR;
  const int kg = dl_slot(lrow, lu % F64DL::UPR, F64DL::UPR);  // the map is its own inverse
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const int64_t ld = side == 0 ? lda : ldb;
    const int r0 = side == 0 ? m0 : n0, rlast = (side == 0 ? M : N) - 1 - r0;
    const char* P = wave_uniform((side == 0 ? A : B) + (int64_t)r0 * ld + k0);
#pragma unroll
    for (int j = 0; j < F64DL::CPO; ++j) {
      const int base_u = (j * (F64Tile::THREADS / 64) + wave) * 64;
      const uint32_t row = (uint32_t)min(lrow + j * (F64Tile::THREADS / F64DL::UPR), rlast);
      uint32_t off = (row * (uint32_t)ld + (uint32_t)(kg * 2)) * 8u;
      asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
      __builtin_amdgcn_global_load_lds((global_void_ptr)(P + off),
                                       (lds_void_ptr)(stage + ((side == 0 ? 0 : F64DL::AU) + base_u) * 16), 16, 0,
                                       0);
    }
  }
}

// Which 16 x 16 MFMA blocks a wave of a 128 x 128 float64 tile computes.  In
// a diagonal tile (m0 == n0, the symmetric products keep only its upper
// triangle) the wave at (1, 0) lies wholly below the diagonal and the waves
// at (0, 0) and (1, 1) hold 6 blocks below it (rb > cb): their results are
// never stored, so the waves skip those MFMAs and the wave of the other
// workgroup on the same SIMD gets the cycles.
enum F64Blocks { kF64All = 0, kF64Upper = 1, kF64None = 2 };
__device__ __forceinline__ int f64_block_mode(bool diag_tile, int wm, int wn) {
  const int m = !diag_tile || wm < wn ? kF64All : wm == wn ? kF64Upper : kF64None;
  return __builtin_amdgcn_readfirstlane(m);  // wave-uniform
}
// The MFMAs of one 2-deep k step; blocks below the diagonal (rb > cb) only
// when `full` (wave-uniform: a branch per block, not a second copy of the
// sequence, which would double the live registers).
__device__ __forceinline__ void f64_mfma_blocks(const v2d (&a)[4], const v2d (&b)[4], v4d (&acc)[4][4], bool full) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        if (rb <= cb || full) acc[rb][cb] = mfma_f64_16x16x4(a[rb][i], b[cb][i], acc[rb][cb]);
}

struct F64Frag {
  v2d a[4], b[4];
};

__device__ __forceinline__ void f64dl_read(const unsigned char* __restrict__ st, int h, F64Frag& f, int lane, int wm,
                                           int wn) {
  const unsigned char* As = st;
  const unsigned char* Bs = st + F64DL::AU * 16;
  const int kg = (lane >> 4) * 2 + h;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = wm * 64 + rb * 16 + (lane & 15);
    f.a[rb] = *reinterpret_cast<const v2d*>(As + (r * F64DL::UPR + dl_slot(r, kg, F64DL::UPR)) * 16);
  }
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int r = wn * 64 + cb * 16 + (lane & 15);
    f.b[cb] = *reinterpret_cast<const v2d*>(Bs + (r * F64DL::UPR + dl_slot(r, kg, F64DL::UPR)) * 16);
  }
}

__device__ __forceinline__ void f64dl_chunk(const unsigned char* __restrict__ st, v4d (&acc)[4][4], int lane, int wm,
                                            int wn, int mode) {
  const unsigned char* As = st;
  const unsigned char* Bs = st + F64DL::AU * 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kg = (lane >> 4) * 2 + h;
    v2d a[4], b[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = wm * 64 + rb * 16 + (lane & 15);
      a[rb] = *reinterpret_cast<const v2d*>(As + (r * F64DL::UPR + dl_slot(r, kg, F64DL::UPR)) * 16);
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int r = wn * 64 + cb * 16 + (lane & 15);
      b[cb] = *reinterpret_cast<const v2d*>(Bs + (r * F64DL::UPR + dl_slot(r, kg, F64DL::UPR)) * 16);
    }
    f64_mfma_blocks(a, b, acc, mode == kF64All);
  }
}

__device__ __forceinline__ void f64dl_nt_tile(const double* __restrict__ A, int64_t lda, const double* __restrict__ B,
                                              int64_t ldb, int M, int N, int K, int m0, int n0,
                                              unsigned char* __restrict__ lds, v4d (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rb][cb][v] = 0.0;
  const int nch = K / F64DL::BK;
  const int mode = f64_block_mode(m0 == n0, wm, wn);
  // Fragment reads one half-chunk ahead, across chunk boundaries too: the
  // reads of the next half are issued before this half's products (the same
  // scheme as the wide split-fp16 core).
  F64Frag f0, f1;
  if (nch > 0) {
    f64dl_issue(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nch > 1) f64dl_issue(A, lda, B, ldb, M, N, m0, n0, F64DL::BK, lds + F64DL::STAGE_BYTES, wave, lane);
    f64dl_read(lds, 0, f0, lane, wm, wn);
  }
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = c + s;
      if (cc < nch) {
        unsigned char* st = lds + s * F64DL::STAGE_BYTES;
        f64dl_read(st, 1, f1, lane, wm, wn);
        if (mode != kF64None) f64_mfma_blocks(f0.a, f0.b, acc, mode == kF64All);
        wait_lgkmcnt0();
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // stage s is free, chunk cc + 1 is in stage s ^ 1
        asm volatile("" ::: "memory");
        if (cc + 2 < nch) f64dl_issue(A, lda, B, ldb, M, N, m0, n0, (cc + 2) * F64DL::BK, st, wave, lane);
        // (after the last chunk this reads a stale stage; those fragments are never used)
        f64dl_read(lds + (s ^ 1) * F64DL::STAGE_BYTES, 0, f0, lane, wm, wn);
        if (mode != kF64None) f64_mfma_blocks(f1.a, f1.b, acc, mode == kF64All);
      }
    }
  }
  __syncthreads();  // no wave leaves (or reuses the LDS) while another may still read the last stage
  return;
  if (nch > 0) f64dl_issue(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (c + s < nch) {
        wait_vmcnt<0>();  // this wave's copies of chunk c + s have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and every wave's; stage s ^ 1 is free
        asm volatile("" ::: "memory");
        if (c + s + 1 < nch)
          f64dl_issue(A, lda, B, ldb, M, N, m0, n0, (c + s + 1) * F64DL::BK, lds + (s ^ 1) * F64DL::STAGE_BYTES, wave,
                      lane);
        if (mode != kF64None) f64dl_chunk(lds + s * F64DL::STAGE_BYTES, acc, lane, wm, wn, mode);
      }
    }
  }
  __syncthreads();  // no wave leaves (or reuses the LDS) while another may still read the last stage
}

// Gram products of float32 data on the float64 matrix cores, operands copied
// straight into LDS as float32 (half the bytes of the widened copy, so NST
// stages of 16 KB fit) and widened to float64 after the fragment read.
//   RIGHT = false (G G^T): element (i, k) at G[i * ld + k]; chunk rows of 16
//     floats (four 16-byte units, dl_slot order); a lane reads the unit
//     holding k = 4 (lane / 16) + q, q = 0..3, with one 128-bit read.
//   RIGHT = true (G^T G): element (i, k) at G[k * ld + i]; the chunk is 16
//     rows k of 128 floats (32 units of four consecutive i), unit u of row k
//     in slot u ^ (4 ((k / 4) % 4)), so the four rows k = 4g + q that one
//     32-bit read touches (g = lane / 16) fall on distinct banks.
// MFMA q of a chunk takes k = 4 (lane / 16) + q, the order of f64_tile, so
// both cores agree bitwise.  Preconditions (checked by the caller): K a
// multiple of 16, ld a multiple of 4 and G 16-byte aligned, and for RIGHT d
// a multiple of 4.  Rows (or columns) beyond d are read from the last ones:
// they only feed outputs that are never stored.  As in f64dl_nt_tile, blocks
// of a diagonal tile wholly below the diagonal are left at zero.
template <bool RIGHT, int NST>
struct F64G {
  static constexpr int BK = 16;
  static constexpr int OPB = 128 * BK * 4;  // bytes per operand and stage
  static constexpr int STAGE_BYTES = 2 * OPB;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int CPO = OPB / 16 / F64Tile::THREADS;  // copies per lane and operand
  static constexpr int PER = 2 * CPO;                      // copies per lane and chunk
  static_assert(NST >= 2 && NST <= 4 && CPO * 16 * F64Tile::THREADS == OPB, "stages, copies cover the chunk");
};

__device__ __forceinline__ int f64g_tslot(int k, int u) { return u ^ (((k >> 2) & 3) << 2); }

template <bool RIGHT, int NST>
__device__ __forceinline__ void f64g_issue(const float* __restrict__ G, int64_t ld, int d, int m0, int n0, int k0,
                                           unsigned char* stage, int wave, int lane) {
  using C = F64G<RIGHT, NST>;
#pragma unroll
  for (int j = 0; j < 2 * C::CPO; ++j) {
    const bool isA = j < C::CPO;
    const int base_u = ((isA ? j : j - C::CPO) * (F64Tile::THREADS / 64) + wave) * 64;
    const int p = base_u + lane;  // unit position inside the operand's chunk
    const int r0 = isA ? m0 : n0;
    // scalar base plus a 32-bit lane byte offset within the chunk: one copy
    // instruction each
    const char* P;
    uint32_t off;
    if constexpr (!RIGHT) {
      const int row = p / 4;
      const int kg = dl_slot(row, p % 4, 4);  // the map is its own inverse
      P = wave_uniform(G + (int64_t)r0 * ld + k0);
      off = ((uint32_t)min(row, d - 1 - r0) * (uint32_t)ld + (uint32_t)(kg * 4)) * 4u;
    } else {
      const int k = p / 32;
      const int u = f64g_tslot(k, p % 32);  // an involution in the unit index too
      P = wave_uniform(G + (int64_t)k0 * ld);
      off = ((uint32_t)k * (uint32_t)ld + (uint32_t)min(r0 + 4 * u, d - 4)) * 4u;
    }
    asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
    __builtin_amdgcn_global_load_lds((global_void_ptr)(P + off),
                                     (lds_void_ptr)(stage + (isA ? 0 : C::OPB) + base_u * 16), 16, 0, 0);
  }
}

template <bool RIGHT, int NST>
__device__ __forceinline__ void f64g_chunk(const unsigned char* __restrict__ st, v4d (&acc)[4][4], int lane, int wm,
                                           int wn, int mode) {
  using C = F64G<RIGHT, NST>;
  const unsigned char* As = st;
  const unsigned char* Bs = st + C::OPB;
  const int g = lane >> 4;
  v4f a[4], b[4];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const bool isA = blk < 4;
    const int i = (isA ? wm : wn) * 64 + (blk & 3) * 16 + (lane & 15);
    const unsigned char* base = isA ? As : Bs;
    v4f v;
    if constexpr (!RIGHT) {
      v = *reinterpret_cast<const v4f*>(base + (i * 4 + dl_slot(i, g, 4)) * 16);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = 4 * g + q;
        v[q] = *reinterpret_cast<const float*>(base + (k * 32 + f64g_tslot(k, i >> 2)) * 16 + (i & 3) * 4);
      }
    }
    if (isA)
      a[blk & 3] = v;
    else
      b[blk & 3] = v;
  }
  const bool full = mode == kF64All;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        if (rb <= cb || full) acc[rb][cb] = mfma_f64_16x16x4((double)a[rb][q], (double)b[cb][q], acc[rb][cb]);
}

template <bool RIGHT, int NST>
__device__ __forceinline__ void f64g_tile(const float* __restrict__ G, int64_t ld, int d, int K, int m0, int n0,
                                          unsigned char* __restrict__ lds, v4d (&acc)[4][4]) {
  using C = F64G<RIGHT, NST>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rb][cb][v] = 0.0;
  const int nch = K / C::BK;
  const int mode = f64_block_mode(m0 == n0, wm, wn);
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nch) f64g_issue<RIGHT, NST>(G, ld, d, m0, n0, s * C::BK, lds + s * C::STAGE_BYTES, wave, lane);
  for (int c0 = 0; c0 < nch; c0 += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const int c = c0 + s;
      if (c < nch) {
        // chunks issued after c and still allowed in flight
        const int after = min(NST - 2, nch - 1 - c);
        if (after >= 2)  // this wave's copies of chunk c have landed
          wait_vmcnt<2 * C::PER>();
        else if (after == 1)
          wait_vmcnt<C::PER>();
        else
          wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and every wave's; the stage of chunk c - 1 is free
        asm volatile("" ::: "memory");
        if (c + NST - 1 < nch)
          f64g_issue<RIGHT, NST>(G, ld, d, m0, n0, (c + NST - 1) * C::BK,
                                 lds + ((s + NST - 1) % NST) * C::STAGE_BYTES, wave, lane);
        if (mode != kF64None) f64g_chunk<RIGHT, NST>(lds + s * C::STAGE_BYTES, acc, lane, wm, wn, mode);
      }
    }
  }
  __syncthreads();  // no wave leaves (or reuses the LDS) while another may still read the last stage
}

// Direct-to-LDS core for float64 operands where its preconditions hold
// (VEC 2: 16-byte aligned rows), else the register-staged one.
template <int VEC>
__device__ __forceinline__ void f64_nt_tile_auto(const double* __restrict__ A, int64_t lda,
                                                 const double* __restrict__ B, int64_t ldb, int M, int N, int K,
                                                 int m0, int n0, double* __restrict__ lds, v4d (&acc)[4][4]) {
  static_assert(F64DL::LDS_BYTES <= (int)sizeof(double) * F64Tile::LDS_DOUBLES, "both cores fit the same LDS");
  if (VEC == 2 && K % F64DL::BK == 0)
    f64dl_nt_tile(A, lda, B, ldb, M, N, K, m0, n0, reinterpret_cast<unsigned char*>(lds), acc);
  else
    f64_tile<double, false, VEC, double, false, VEC>(A, lda, B, ldb, M, N, K, m0, n0, lds, acc);
}

template <typename F>
__device__ __forceinline__ void f64_for_each(const v4d (&acc)[4][4], F&& f) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        f(wm * 64 + rb * 16 + f64_row(lane, v), wn * 64 + cb * 16 + (lane & 15), acc[rb][cb][v]);
}

}  // namespace mr
