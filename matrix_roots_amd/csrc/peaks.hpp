// Register-only MFMA loops that measure the matrix-core rates a kernel of
// this library can reach, next to the peaks derived from the device's
// compute-unit count and clock.
#pragma once

#include <hip/hip_runtime.h>

namespace mr {

enum PeakKind { kPeakF32 = 0, kPeakF64 = 1, kPeakF16 = 2, kPeakI8 = 3 };
constexpr int kPeakKinds = 4;

// Dense MFMA flops (int8: operations) per clock per compute unit on gfx950
// (4 SIMDs).
constexpr double kMfmaFlopsPerClockCU[kPeakKinds] = {256.0, 128.0, 4096.0, 8192.0};

// Launch `blocks` workgroups of 256 threads, each wave running `iters`
// rounds of independent MFMA chains of the kind, on fixed small operands or
// (random) on per-lane random ones; returns the flops one such launch
// performs through *flops.
hipError_t launch_peak_loop(int kind, int blocks, int iters, bool random, double* flops, hipStream_t s);

}  // namespace mr
