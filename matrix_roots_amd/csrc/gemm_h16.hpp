// C = A * B^T on the fp16 matrix cores with float32 accumulation, for
// operands stored as fp16 arrays (the hi half of the split storage): one
// v_mfma_f32_32x32x16_f16 per 32 x 32 x 16 block.
//
// Two cores over one block-shape description (H16Shape: BM x BN block tile,
// WM x WN waves, each wave (BM / WM) x (BN / WN) in 32 x 32 MFMA blocks).
// A and B rows are K-contiguous ("NT"), so both operand panels are read
// along rows and staged the same way:
//   * h16g_nt_tile: register-staged, K in chunks of BK through two padded LDS
//     stages with one barrier per chunk (any size and alignment);
//   * h16dl_nt_tile: direct global -> LDS copies, unpadded XOR-swizzled rows,
//     K-chunks of 64 (contraction a multiple of 64, 16-byte rows).
#pragma once

#include "mr_common.hpp"

namespace mr {

// ------------------------------------------------------------ block shapes
// BM x BN block tile, WM x WN waves, each wave (BM / WM) x (BN / WN) in 32 x 32
// MFMA blocks (RB x CB of them), K in chunks of BK through two LDS stages.
// H16Shape<128, 128, 2, 2> (256 threads, two blocks per CU) and
// H16Shape<256, 256, 2, 4> (512 threads, 128 accumulator registers per lane,
// one block and two waves per SIMD: each operand panel read half as often)
// are the shapes in use.
template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64>
struct H16Shape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int RB = BM / WM / 32, CB = BN / WN / 32;
  static constexpr int BK = BK_, PAD = 8, LDW = BK + PAD;
  static constexpr int AARR = BM * LDW, BARR = BN * LDW;
  static constexpr int STAGE = AARR + BARR;
  static constexpr int LDS_HALVES = 2 * STAGE;
};

template <class S, int ROWS, int VEC>
struct H16GLoader {
  static constexpr int GPR = S::BK / 8;
  static constexpr int PER = (ROWS * S::BK) / (S::THREADS * 8);
  static_assert(PER * S::THREADS * 8 == ROWS * S::BK, "loader covers the chunk");
  v8h r[PER];

  __device__ __forceinline__ void load(const _Float16* __restrict__ P, int64_t ld, int rows, int K, int r0, int k0,
                                       int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int row, grp;
      tile_slot<GPR>(tid + p * S::THREADS, row, grp);
      const int gr = r0 + row, gk = k0 + grp * 8;
      const int64_t off = (int64_t)gr * ld + gk;
      if constexpr (VEC == 8) {
        v8h h = {};
        if (gr < rows && gk < K) h = *reinterpret_cast<const v8h*>(P + off);
        r[p] = h;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[p][e] = (gr < rows && gk + e < K) ? P[off + e] : (_Float16)0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(_Float16* __restrict__ dst, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int row, grp;
      tile_slot<GPR>(tid + p * S::THREADS, row, grp);
      *reinterpret_cast<v8h*>(dst + row * S::LDW + grp * 8) = r[p];
    }
  }
};

template <class S>
__device__ __forceinline__ void h16g_chunk(const _Float16* __restrict__ st, v16f (&acc)[S::RB][S::CB], int lane,
                                           int wm, int wn) {
  const _Float16* As = st;
  const _Float16* Bs = st + S::AARR;
  const int koff = (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < S::BK / 16; ++ks) {
    v8h a[S::RB], b[S::CB];
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb)
      a[rb] = *reinterpret_cast<const v8h*>(As + (wm * (S::BM / S::WM) + rb * 32 + (lane & 31)) * S::LDW + ks * 16 +
                                            koff);
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
      b[cb] = *reinterpret_cast<const v8h*>(Bs + (wn * (S::BN / S::WN) + cb * 32 + (lane & 31)) * S::LDW + ks * 16 +
                                            koff);
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb) acc[rb][cb] = mfma_f16_32x32x16(a[rb], b[cb], acc[rb][cb]);
  }
}

// acc = A[m0:m0+BM, :K] * B[n0:n0+BN, :K]^T (rows beyond M / N and columns
// beyond K read as zero), per-wave blocks laid out as in h16g_for_each.
template <class S, int VEC>
__device__ __forceinline__ void h16g_nt_tile(const _Float16* __restrict__ A, int64_t lda,
                                             const _Float16* __restrict__ B, int64_t ldb, int M, int N, int K, int m0,
                                             int n0, _Float16* __restrict__ lds, v16f (&acc)[S::RB][S::CB]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;
  H16GLoader<S, S::BM, VEC> la;
  H16GLoader<S, S::BN, VEC> lb;
  la.load(A, lda, M, K, m0, 0, tid);
  lb.load(B, ldb, N, K, n0, 0, tid);
  la.store(lds, tid);
  lb.store(lds + S::AARR, tid);
  __syncthreads();
  int stage = 0;
  for (int k0 = 0; k0 < K; k0 += S::BK) {
    const bool more = k0 + S::BK < K;
    if (more) {
      la.load(A, lda, M, K, m0, k0 + S::BK, tid);
      lb.load(B, ldb, N, K, n0, k0 + S::BK, tid);
    }
    h16g_chunk<S>(lds + stage * S::STAGE, acc, lane, wm, wn);
    if (more) {
      _Float16* nxt = lds + (stage ^ 1) * S::STAGE;
      la.store(nxt, tid);
      lb.store(nxt + S::AARR, tid);
    }
    __syncthreads();
    stage ^= 1;
  }
}

// Visit every accumulator element as (row, col) local to the block tile.
template <class S, typename F>
__device__ __forceinline__ void h16g_for_each(const v16f (&acc)[S::RB][S::CB], F&& f) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        f(wm * (S::BM / S::WM) + rb * 32 + f32_row(lane, v), wn * (S::BN / S::WN) + cb * 32 + (lane & 31),
          acc[rb][cb][v]);
}

// ------------------------------------------- direct-to-LDS core (fp16 only)
// The same block tile and wave layout as H16Shape<BM, BN, WM, WN>, with the
// operand chunks copied from global memory straight into LDS by
// global_load_lds_dwordx4 (no staging registers, no LDS store instructions):
// each instruction moves 16 bytes per lane into 1 KB of consecutive LDS.  A
// chunk row is BK halves (UPR 16-byte units, no padding); the unit of k-group
// kg of row r sits in slot kg ^ ((r / (16 / UPR)) % UPR), so the 16 lanes of
// one LDS read cycle (16 consecutive rows, same k-group) hit 16 distinct
// 16-byte bank groups.  Two stages; a wave waits for its own copies of the
// next chunk (vmcnt) and a plain s_barrier publishes them, which leaves the
// copies of the chunk after in flight during the MFMAs.
//
// Preconditions (checked by the caller): K a multiple of BK, lda and ldb
// multiples of 8, A and B 16-byte aligned.  Rows beyond M or N are read from
// row M - 1 or N - 1: they only feed outputs that are never stored.
template <int BM_, int BN_, int WM_, int WN_, int BK_>
struct H16DLShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr int THREADS = 64 * WM * WN, NW = WM * WN;
  static constexpr int RB = BM / WM / 32, CB = BN / WN / 32;
  static constexpr int UPR = BK / 8;
  static constexpr int AU = BM * UPR, BU = BN * UPR;  // 16-byte units per stage
  static constexpr int STAGE_BYTES = (AU + BU) * 16;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int NA = AU / (64 * NW), NB = BU / (64 * NW);  // copies per wave per chunk
  static_assert(NA * 64 * NW == AU && NB * 64 * NW == BU, "copies cover the chunk");
  static_assert(UPR == 4 || UPR == 8, "swizzle period");
};


template <class S>
__device__ __forceinline__ void h16dl_issue(const _Float16* __restrict__ A, int64_t lda, const _Float16* __restrict__ B,
                                            int64_t ldb, int M, int N, int m0, int n0, int k0, unsigned char* stage,
                                            int wave, int lane) {
#pragma unroll
  for (int j = 0; j < S::NA + S::NB; ++j) {
    const bool isA = j < S::NA;
    const int base_u = ((isA ? j : j - S::NA) * S::NW + wave) * 64;
    const int u = base_u + lane;
    const int row = u / S::UPR;
    const int kg = dl_slot(row, u % S::UPR, S::UPR);  // the map is its own inverse
    // scalar base (row m0 or n0, column k0) plus a 32-bit lane byte offset
    // within the tile's rows: one copy instruction each
    const char* P = wave_uniform(isA ? A + (int64_t)m0 * lda + k0 : B + (int64_t)n0 * ldb + k0);
    uint32_t off = ((uint32_t)min(row, isA ? M - 1 - m0 : N - 1 - n0) * (uint32_t)(isA ? lda : ldb) +
                    (uint32_t)(kg * 8)) * 2u;
    asm volatile("" : "+v"(off));  // opaque per copy: the offset stays a 32-bit lane value
    __builtin_amdgcn_global_load_lds((global_void_ptr)(P + off),
                                     (lds_void_ptr)(stage + (isA ? 0 : S::AU * 16) + base_u * 16), 16, 0, 0);
  }
}

template <class S>
__device__ __forceinline__ void h16dl_chunk(const unsigned char* __restrict__ st, v16f (&acc)[S::RB][S::CB], int wm,
                                            int wn, int lane) {
  const unsigned char* As = st;
  const unsigned char* Bs = st + S::AU * 16;
#pragma unroll
  for (int ks = 0; ks < S::BK / 16; ++ks) {
    v8h a[S::RB], b[S::CB];
    const int kg = ks * 2 + (lane >> 5);
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb) {
      const int r = wm * (S::BM / S::WM) + rb * 32 + (lane & 31);
      a[rb] = *reinterpret_cast<const v8h*>(As + (r * S::UPR + dl_slot(r, kg, S::UPR)) * 16);
    }
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb) {
      const int r = wn * (S::BN / S::WN) + cb * 32 + (lane & 31);
      b[cb] = *reinterpret_cast<const v8h*>(Bs + (r * S::UPR + dl_slot(r, kg, S::UPR)) * 16);
    }
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb) acc[rb][cb] = mfma_f16_32x32x16(a[rb], b[cb], acc[rb][cb]);
  }
}

// One k-step's fragments of a wave, the reads that fill them, the products
// that use them, and the instruction order for a region that holds one
// k-step's products and the next k-step's reads (reads spread evenly).
template <class S>
struct H16Frag {
  v8h a[S::RB], b[S::CB];
};

template <class S>
__device__ __forceinline__ void h16dl_read(const unsigned char* __restrict__ st, int ks, H16Frag<S>& f, int wm,
                                           int wn, int lane) {
  const unsigned char* As = st;
  const unsigned char* Bs = st + S::AU * 16;
  const int kg = ks * 2 + (lane >> 5);
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb) {
    const int r = wm * (S::BM / S::WM) + rb * 32 + (lane & 31);
    f.a[rb] = *reinterpret_cast<const v8h*>(As + (r * S::UPR + dl_slot(r, kg, S::UPR)) * 16);
  }
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) {
    const int r = wn * (S::BN / S::WN) + cb * 32 + (lane & 31);
    f.b[cb] = *reinterpret_cast<const v8h*>(Bs + (r * S::UPR + dl_slot(r, kg, S::UPR)) * 16);
  }
}

template <class S>
__device__ __forceinline__ void h16dl_mfma(const H16Frag<S>& f, v16f (&acc)[S::RB][S::CB]) {
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb) acc[rb][cb] = mfma_f16_32x32x16(f.a[rb], f.b[cb], acc[rb][cb]);
}

template <class S>
__device__ __forceinline__ void h16dl_sched_overlap() {
  constexpr int NR = S::RB + S::CB, NM = S::RB * S::CB;
  constexpr int PER = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // products
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
  }
  if (NM > PER * NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR, 0);
}

// acc = A[m0:m0+BM, :K] * B[n0:n0+BN, :K]^T in the accumulator layout of
// h16g_for_each for the H16Shape of the same BM, BN, WM, WN.
template <class S>
__device__ __forceinline__ void h16dl_nt_tile(const _Float16* __restrict__ A, int64_t lda,
                                              const _Float16* __restrict__ B, int64_t ldb, int M, int N, int K, int m0,
                                              int n0, unsigned char* __restrict__ lds, v16f (&acc)[S::RB][S::CB]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS offsets
  const int wm = wave / S::WN, wn = wave % S::WN;
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;
  const int nch = K / S::BK;
  // Fragment reads one k-step ahead, across chunk boundaries too (the scheme
  // of the wide split-fp16 Newton core): the barrier sits before the last
  // k-step's products, once every wave has finished reading the stage (LDS
  // count 0) and holds the next chunk's copies (vector-memory count 0).
  constexpr int KS = S::BK / 16;
  static_assert(KS % 2 == 0, "an even number of k-steps per chunk");
  H16Frag<S> f[2];
  if (nch > 0) {
    h16dl_issue<S>(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (nch > 1) h16dl_issue<S>(A, lda, B, ldb, M, N, m0, n0, S::BK, lds + S::STAGE_BYTES, wave, lane);
    h16dl_read<S>(lds, 0, f[0], wm, wn, lane);
  }
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int cc = c + s;
      if (cc < nch) {
        unsigned char* st = lds + s * S::STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
          h16dl_read<S>(st, ks + 1, f[(ks + 1) & 1], wm, wn, lane);
          h16dl_mfma<S>(f[ks & 1], acc);
          h16dl_sched_overlap<S>();
        }
        wait_lgkmcnt0();
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // stage s is free, chunk cc + 1 is in stage s ^ 1
        asm volatile("" ::: "memory");
        if (cc + 2 < nch) h16dl_issue<S>(A, lda, B, ldb, M, N, m0, n0, (cc + 2) * S::BK, st, wave, lane);
        // (after the last chunk this reads a stale stage; those fragments are never used)
        h16dl_read<S>(lds + (s ^ 1) * S::STAGE_BYTES, 0, f[0], wm, wn, lane);
        h16dl_mfma<S>(f[(KS - 1) & 1], acc);
        h16dl_sched_overlap<S>();
      }
    }
  }
  __syncthreads();  // no wave leaves while another may still read the last stage
  return;
  if (nch > 0) h16dl_issue<S>(A, lda, B, ldb, M, N, m0, n0, 0, lds, wave, lane);
  for (int c = 0; c < nch; c += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (c + s < nch) {
        wait_vmcnt<0>();  // this wave's copies of chunk c + s have landed
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // ... and every wave's; stage s ^ 1 is free
        asm volatile("" ::: "memory");
        if (c + s + 1 < nch)
          h16dl_issue<S>(A, lda, B, ldb, M, N, m0, n0, (c + s + 1) * S::BK, lds + (s ^ 1) * S::STAGE_BYTES, wave,
                         lane);
        h16dl_chunk<S>(lds + s * S::STAGE_BYTES, acc, wm, wn, lane);
      }
    }
  }
  __syncthreads();  // no wave leaves while another may still read the last stage
}

// The direct-to-LDS tile of an H16Shape (K-chunks of 64) and the LDS bytes a
// kernel needs for either core.
template <class S>
using H16DLOf = H16DLShape<S::BM, S::BN, S::WM, S::WN, 64>;
template <class S>
constexpr int h16_lds_bytes() {
  return (H16DLOf<S>::LDS_BYTES > 2 * S::LDS_HALVES) ? H16DLOf<S>::LDS_BYTES : 2 * S::LDS_HALVES;
}
// ... or the wide-store epilogue's slabs (17 KB per wave), whichever is larger
template <class S>
constexpr int h16_kernel_lds_bytes(int slab_bytes_per_wave) {
  return h16_lds_bytes<S>() > slab_bytes_per_wave * (S::THREADS / 64) ? h16_lds_bytes<S>()
                                                                       : slab_bytes_per_wave * (S::THREADS / 64);
}

// Direct-to-LDS core where its preconditions hold (VEC 8 implies 16-byte
// aligned operands with leading dimensions multiple of 8), else the
// register-staged one.
template <class S, int VEC>
__device__ __forceinline__ void h16_nt_tile_auto(const _Float16* __restrict__ A, int64_t lda,
                                                 const _Float16* __restrict__ B, int64_t ldb, int M, int N, int K,
                                                 int m0, int n0, unsigned char* __restrict__ lds,
                                                 v16f (&acc)[S::RB][S::CB]) {
  if (VEC == 8 && K % 64 == 0)
    h16dl_nt_tile<H16DLOf<S>>(A, lda, B, ldb, M, N, K, m0, n0, lds, acc);
  else
    h16g_nt_tile<S, VEC>(A, lda, B, ldb, M, N, K, m0, n0, reinterpret_cast<_Float16*>(lds), acc);
}

}  // namespace mr
