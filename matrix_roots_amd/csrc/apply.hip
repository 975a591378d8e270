// Two-sided application of the quarter powers on the fp16 matrix cores.
//
//   U = alpha * XL * G * XR
//
// (marin.community, "Sharding EMA-Gram eigensolves", section "Background":
// the inverse quarter powers shape the update direction; the two-sided form
// is Shampoo's, tilderesearch "Online KL Shampoo", section 1.)
// Both products run as C = A * B^T on row-contiguous split operands:
//   W^T = XR^T * G^T  (n x m; A = rows of XR^T, B = G rows, contraction n)
//   U   = XL * W      (m x n; A = XL rows, B = W^T rows, contraction m)
// XR's split copy is written transposed, so no symmetry of XR is assumed
// (the roots this library produces are symmetric to the last bit, and for
// them the transposed copy is bitwise the plain one).  The host runtime
// issues the launches.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace mr {

// ---------------------------------------------------------- split-fp16 apply
// The same two products on the fp16 matrix cores with split operands
// (float32-accurate, x3dl_nt_tile).  Each float32 operand is first scaled by
// a power of two 2^s that puts its largest magnitude in [2^14, 2^15)
// (absmax_kernel, then split_pad_kernel): the scaling is exact, keeps both
// fp16 halves clear of overflow and of the subnormal range for any input
// scale, and makes the result exactly equivariant under power-of-two
// scalings of the inputs.  Rows are padded with zeros to a multiple of 32
// (the zeros add nothing and make every contraction whole 32-deep chunks).
// W^T = XR^T G^T goes through float32 and is split with its own scale before
// U = alpha XL W; each product multiplies by 2^-(s_A + s_B).

// Scale exponent of a matrix from its largest magnitude (float32 bits):
// 2^s max in [2^14, 2^15) (s clamped to [-126, 126] so that 2^s and 2^-s stay
// float32 normals: only a maximum below 2^-112, float32's subnormal range,
// lands lower); 0 for an all-zero or non-finite maximum.
__device__ __forceinline__ int split_scale_exp(const uint32_t* amax) {
  const float m = __uint_as_float(*amax);
  if (!(m > 0.f) || !isfinite(m)) return 0;
  return max(-126, min(126, 14 - ilogbf(m)));
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int32_t n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void absmax_kernel(const AbsMaxBatch batch) {
  __shared__ uint32_t red[256];
  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const AbsMaxJob& J = batch.job[jx];
  const int64_t r0 = (b - J.block_begin) * kAbsMaxRows;
  const int64_t r1 = min((int64_t)J.rows, r0 + kAbsMaxRows);
  uint32_t m = 0u;  // bits of a non-negative float (a NaN's exceed infinity's)
  for (int64_t r = r0; r < r1; ++r) {
    const float* row = J.src + r * J.lds;
    if (J.vec4) {
      for (int c = threadIdx.x * 4; c < J.cols; c += 1024) {
        const v4f v = *reinterpret_cast<const v4f*>(row + c);
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, __float_as_uint(fabsf(v[k])));
      }
    } else {
      for (int c = threadIdx.x; c < J.cols; c += 256) m = max(m, __float_as_uint(fabsf(row[c])));
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(J.amax, red[0]);
}

// 2048 padded elements per workgroup, 8 per lane (ldd is a multiple of 8, so
// a lane's 8 never straddle rows).
__global__ __launch_bounds__(256) void split_pad_kernel(const SplitPadBatch batch) {
  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const SplitPadJob& J = batch.job[jx];
  const int64_t e = (b - J.block_begin) * 2048 + threadIdx.x * 8;
  const int64_t total = (int64_t)J.rows * J.ldd;
  if (e >= total) return;
  const int64_t row = e / J.ldd;
  const int col = (int)(e - row * J.ldd);
  const float scale = ldexpf(1.0f, split_scale_exp(J.amax));
  float v[8];
  const float* src = J.src + row * J.lds + col;
  if (J.vec4 && col + 8 <= J.cols) {
    const v4f x = *reinterpret_cast<const v4f*>(src), y = *reinterpret_cast<const v4f*>(src + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = x[k];
      v[k + 4] = y[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = col + k < J.cols ? src[k] : 0.0f;
  }
  v8h h, l;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    _Float16 a, c;
    split_f32(v[k] * scale, a, c);
    h[k] = a;
    l[k] = c;
  }
  *reinterpret_cast<v8h*>(J.dst + e) = h;
  *reinterpret_cast<v8h*>(J.dst + total + e) = l;
}

// Transposed split copy: dst (rows x ldd) row r = src column r, for 64 x 64
// dst tiles; the tile's src rows are read coalesced into LDS, then each lane
// writes 8 consecutive dst elements of one row (16-byte hi and lo stores).
// dst columns at or past cols (src rows that do not exist) are zero.
__global__ __launch_bounds__(256) void split_pad_t_kernel(const SplitPadBatch batch) {
  __shared__ float t[64][65];
  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const SplitPadJob& J = batch.job[jx];
  const int tiles_c = (int)((J.ldd + 63) / 64);
  const int blk = (int)(b - J.block_begin);
  const int r0 = (blk / tiles_c) * 64;  // dst rows = src columns
  const int c0 = (blk % tiles_c) * 64;  // dst columns = src rows
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int i = grp + 4 * e;  // src row c0 + i, src column r0 + lane
    const int sr = c0 + i, sc = r0 + lane;
    t[i][lane] = (sr < J.cols && sc < J.rows) ? J.src[(int64_t)sr * J.lds + sc] : 0.0f;
  }
  __syncthreads();
  const float scale = ldexpf(1.0f, split_scale_exp(J.amax));
  const int64_t total = (int64_t)J.rows * J.ldd;
  const int b0 = (threadIdx.x & 7) * 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int a = (threadIdx.x >> 3) + 32 * h;
    const int dr = r0 + a, dc = c0 + b0;
    if (dr >= J.rows || dc >= J.ldd) continue;
    v8h hi, lo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      _Float16 x, y;
      split_f32(t[b0 + k][a] * scale, x, y);
      hi[k] = x;
      lo[k] = y;
    }
    const int64_t e = (int64_t)dr * J.ldd + dc;
    *reinterpret_cast<v8h*>(J.dst + e) = hi;
    *reinterpret_cast<v8h*>(J.dst + total + e) = lo;
  }
}

__global__ __launch_bounds__(256, 2) void x3_apply_kernel(const X3ApplyBatch batch) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[X3DL::LDS_BYTES];
  const int64_t b = blockIdx.x;
  int jx = 0;
  while (jx + 1 < batch.njobs && b >= batch.job[jx + 1].block_begin) ++jx;
  const X3ApplyJob& J = batch.job[jx];
  const int tile = (int)xcd_remap(b - J.block_begin, round8(J.nblocks));
  if (tile >= J.nblocks) return;
  int ti, tj;
  full_tile_grouped(tile, (J.M + X3Tile::BM - 1) / X3Tile::BM, J.tiles_n, ti, tj);
  const int m0 = ti * X3Tile::BM, n0 = tj * X3Tile::BN;
  const int M = J.M, N = J.N;
  const SplitRef A{J.a, J.a + (int64_t)M * J.ld}, Bm{J.b, J.b + (int64_t)N * J.ld};
  v16f acc[2][2];
  x3dl_nt_tile(A, J.ld, Bm, J.ld, M, N, (int)J.ld, m0, n0, smem, acc);
  const float alpha = J.alpha;
  const float fa = ldexpf(1.0f, -split_scale_exp(J.a_max)), fb = ldexpf(1.0f, -split_scale_exp(J.b_max));
  f32_for_each(acc, [&](int r, int c, float v) {
    const int gr = m0 + r, gc = n0 + c;
    if (gr < M && gc < N) J.c[(int64_t)gr * J.ldc + gc] = alpha * v * fa * fb;  // exact powers of two
  });
}

hipError_t launch_fill_zero(uint32_t* p, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(min(64, (n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_absmax(const AbsMaxBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(absmax_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_split_pad(const SplitPadBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_pad_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_split_pad_t(const SplitPadBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_pad_t_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_x3_apply(const X3ApplyBatch& b, hipStream_t s) {
  if (b.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(x3_apply_kernel, dim3(b.total_blocks), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace mr
