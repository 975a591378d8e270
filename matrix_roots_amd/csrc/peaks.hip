// Matrix-core rate probes: each wave keeps its accumulators in registers
// and issues independent MFMA chains back to back, with no memory traffic,
// so the measured rate is what the MFMA pipes deliver at the clock the chip
// sustains under that load.
#include "mr_common.hpp"
#include "peaks.hpp"

namespace mr {

namespace {

// 8 chains of 16 registers for f32 32x32x2, f16 32x32x16 and i8 32x32x32, 16 chains of 8
// registers for f64 16x16x4: with two waves per SIMD that keeps enough
// independent MFMAs in flight to cover each instruction's pipeline latency
// (4 chains reach only 78% of the fp16 rate).
template <int KIND>
struct PeakCfg;
template <>
struct PeakCfg<kPeakF32> {
  static constexpr int CHAINS = 8;
  static constexpr double FLOPS = 2.0 * 32 * 32 * 2;
};
template <>
struct PeakCfg<kPeakF16> {
  static constexpr int CHAINS = 8;
  static constexpr double FLOPS = 2.0 * 32 * 32 * 16;
};
template <>
struct PeakCfg<kPeakI8> {
  static constexpr int CHAINS = 8;
  static constexpr double FLOPS = 2.0 * 32 * 32 * 32;
};
template <>
struct PeakCfg<kPeakF64> {
  static constexpr int CHAINS = 16;
  static constexpr double FLOPS = 2.0 * 16 * 16 * 4;
};

}  // namespace

// Per-lane pseudo-random operand bits (xorshift32 of the workgroup, lane and
// chain), for the loops that draw the power real data draw.
__device__ __forceinline__ uint32_t peak_bits(uint32_t k) {
  uint32_t x = k * 2654435761u + 0x9e3779b9u;
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}
__device__ __forceinline__ float peak_unit(uint32_t k) {  // in [-1, 1)
  return (float)(peak_bits(k) >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

// `sink` is written only when iters < 0, which the host never passes: the
// branch keeps the chains live without any memory access.  RANDOM = 0: every
// chain multiplies the same small operands (what the matrix cores sustain
// at the clock they hold with little switching); 1: each lane and chain its
// own random operands, uniform in [-1, 1) (int8: digits in [-64, 63], as
// the digit planes hold), which draw more power and hold a lower clock.
template <int KIND, int RANDOM>
__global__ __launch_bounds__(256, 2) void peak_kernel(int iters, float* sink) {
  constexpr int C = PeakCfg<KIND>::CHAINS;
  const float x = (float)(threadIdx.x & 63) * (1.0f / 64.0f);
  const uint32_t key = (blockIdx.x * 256u + threadIdx.x) * 64u;
  float total = 0.0f;
  if constexpr (KIND == kPeakF64) {
    v4d acc[C];
    double a[C], b[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[c] = v4d{0.0, 0.0, 0.0, 0.0};
      a[c] = RANDOM ? (double)peak_unit(key + 2 * c) : x;
      b[c] = RANDOM ? (double)peak_unit(key + 2 * c + 1) : 1.0 - x;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = mfma_f64_16x16x4(a[c], b[c], acc[c]);
#pragma unroll
    for (int c = 0; c < C; ++c) total += (float)(acc[c][0] + acc[c][3]);
  } else if constexpr (KIND == kPeakI8) {
    typedef int v4i_ __attribute__((ext_vector_type(4)));
    typedef int v16i_ __attribute__((ext_vector_type(16)));
    v16i_ acc[C];
    v4i_ a[C], b[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // four int8 digits in [-64, 63] per word: bytes of (bits & 0x7f7f7f7f) - 0x40404040
        a[c][e] = RANDOM ? (int)((peak_bits(key + 8 * c + e) & 0x7f7f7f7fu) - 0x40404040u)
                         : (int)(threadIdx.x * 7u + (unsigned)e) & 0x3f3f3f3f;
        b[c][e] = RANDOM ? (int)((peak_bits(key + 8 * c + 4 + e) & 0x7f7f7f7fu) - 0x40404040u)
                         : (int)(threadIdx.x * 3u + 5u * (unsigned)e) & 0x3f3f3f3f;
      }
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c], b[c], acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < C; ++c) total += (float)(acc[c][0] + acc[c][15]);
  } else {
    v16f acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
    if constexpr (KIND == kPeakF32) {
      float a[C], b[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        a[c] = RANDOM ? peak_unit(key + 2 * c) : x;
        b[c] = RANDOM ? peak_unit(key + 2 * c + 1) : 1.0f - x;
      }
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] = mfma_f32_32x32x2(a[c], b[c], acc[c]);
    } else {
      v8h a[C], b[C];
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[c][e] = (_Float16)(RANDOM ? peak_unit(key + 16 * c + e) : x * 0.125f * (float)e);
          b[c][e] = (_Float16)(RANDOM ? peak_unit(key + 16 * c + 8 + e) : 0.5f - x * 0.0625f * (float)e);
        }
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] = mfma_f16_32x32x16(a[c], b[c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) total += acc[c][0] + acc[c][15];
  }
  if (iters < 0) sink[threadIdx.x] = total;
}

hipError_t launch_peak_loop(int kind, int blocks, int iters, bool random, double* flops, hipStream_t s) {
  if (blocks <= 0 || iters <= 0) return hipErrorInvalidValue;
  const double waves = (double)blocks * 4.0 * (double)iters;
  auto go = [&](auto kernel, int chains, double per) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, s, iters, (float*)nullptr);
    *flops = waves * chains * per;
  };
  switch (kind) {
    case kPeakF32:
      if (random)
        go(peak_kernel<kPeakF32, 1>, PeakCfg<kPeakF32>::CHAINS, PeakCfg<kPeakF32>::FLOPS);
      else
        go(peak_kernel<kPeakF32, 0>, PeakCfg<kPeakF32>::CHAINS, PeakCfg<kPeakF32>::FLOPS);
      break;
    case kPeakF64:
      if (random)
        go(peak_kernel<kPeakF64, 1>, PeakCfg<kPeakF64>::CHAINS, PeakCfg<kPeakF64>::FLOPS);
      else
        go(peak_kernel<kPeakF64, 0>, PeakCfg<kPeakF64>::CHAINS, PeakCfg<kPeakF64>::FLOPS);
      break;
    case kPeakF16:
      if (random)
        go(peak_kernel<kPeakF16, 1>, PeakCfg<kPeakF16>::CHAINS, PeakCfg<kPeakF16>::FLOPS);
      else
        go(peak_kernel<kPeakF16, 0>, PeakCfg<kPeakF16>::CHAINS, PeakCfg<kPeakF16>::FLOPS);
      break;
    case kPeakI8:
      if (random)
        go(peak_kernel<kPeakI8, 1>, PeakCfg<kPeakI8>::CHAINS, PeakCfg<kPeakI8>::FLOPS);
      else
        go(peak_kernel<kPeakI8, 0>, PeakCfg<kPeakI8>::CHAINS, PeakCfg<kPeakI8>::FLOPS);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mr
