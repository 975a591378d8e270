// Kernel-argument records shared by the host runtime and the kernels, and the
// launcher functions each kernel file exports to the host runtime.
//
// Per-problem tables travel by value in the kernel arguments (a bounded
// number of records per launch, under the 4 KiB argument limit); the Jacobi
// route copies its records into the caller's workspace with a kernel, so no
// entry point ever copies descriptors with the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/matrix_roots.h"

namespace mr {

constexpr int kMaxSyrkJobs = 48;   // Gram EMA: one launch per side for up to 48 weights (2.3 KiB)
constexpr int kMaxRootJobs = 48;   // root statistics, init and finalize launches (3.1 KiB)
constexpr int kMaxClasses = 8;
constexpr int kJacobiMaxD = 128;
// MR_AUTO takes the eigendecomposition route up to this size.  Measured on
// MI355X per root call, Jacobi against Newton: d = 24: 0.33 / 0.33 ms for 4
// matrices, 0.50 / 0.69 for 256; d = 32: 0.49 / 0.36 and 0.57 / 0.73; d = 48:
// 1.01 / 0.53 and 1.15 / 0.92; d = 128: 9.3 / 1.0.  Up to 32 the eigen route
// costs at most a tenth of a millisecond more on small batches, wins on large
// ones, and its roots are accurate to float64 rounding.
constexpr int kJacobiAutoMaxD = 32;
// Smallest Gram size whose split-fp16 Newton stages take the 256 x 256 tile
// (d a multiple of 32).  Smaller Grams take the 128 x 128 direct-to-LDS tile
// (two workgroups per CU): a d = 128 Gram fills it instead of a quarter of
// the wide one, and the more numerous tiles balance better.  Measured on
// MI355X, one root call: 4 x 128^2 1.41 -> 1.03 ms, 64 x 256^2 1.97 -> 1.52
// ms, 256 x 512^2 12.6 -> 12.2 ms.  In whole weight sets the wide tile's
// fewer operand re-reads win from d = 1536 (128 x 1536^2 + 128 x 3072^2:
// 716 against 759 ms with narrow tiles; 80 x 1024^2 + 16 x 4096^2: 199
// against 208), and the 1024^2 class takes either at the same speed.
constexpr int kWideMinD = 1024;
// Smallest Gram size whose float64 Newton steps take the int8 digit-plane
// products (smaller ones keep the float64 kernel).  Measured on MI355X per
// size class, digit-plane stages (plus the pass that cuts M's planes) against
// the float64 kernel: 512^2 x 256 (ill-conditioned batch) 26.3 + 6.5 against
// 27.9 ms per step of three calls; 1024^2 x 80: 9.0 + 0.5 against 9.8 ms;
// 1536^2 x 128: 17.7 against 23.8 ms; 4096^2 x 16: 77.8 against 98.8 ms.
constexpr int kI8MinD = 1024;
constexpr int kJacobiDefaultSweeps = 30;
constexpr int kJacobiMaxSweeps = 100;
constexpr int kStatsRows = 32;       // rows of A per statistics workgroup (one 32-row tile stripe)
constexpr int kFinalRows = 8;        // rows of X per finalize workgroup
constexpr double kSwitchM = 5e-4;    // float64 -> split-fp16 products once the eigenvalue floor reaches this
constexpr double kNewtonTol = 1e-6;  // stop once 1 - m_K <= this (scalar recurrence)
constexpr double kBoundSafety = 1.01;
// Lowest eigenvalue floor eps / c the Newton launches cover without a rescale
// (below it float64 rounding of M0 already reaches the floor's size).
constexpr double kNoneFloorCap = 1e-16;

// Float64 Newton steps of the default path run their products on int8 digit
// planes (gemm_i8.hpp): kOzSlices planes per matrix, each dp x dp bytes (dp =
// d rounded up to kOzTile), for M, T2 and T4, plus M's row exponents (dp
// int32).  They live in the parts of the five float64 slots of d*d that a
// float64 step leaves idle, where those are 16-byte aligned (d a multiple of
// 4): M's and T4's twelve planes fill the fifth slot (8 d^2 bytes) and the
// second half of the second (4 d^2, a split half-slot no step uses) as far
// as whole planes go; T2's six sit in the slot that will take M' (its float64
// M of the step before is dead, and stage 2 writes M' only once T2 is read),
// when they fit.  The rest, and the exponents, follow the slots.
constexpr int kOzSlices = 6;
constexpr int kOzTile = 128;
constexpr int kOzSliceRows = 16;  // rows per workgroup of the pass that cuts M's planes
__host__ __device__ inline int64_t oz_pad(int64_t d) { return (d + kOzTile - 1) / kOzTile * kOzTile; }
__host__ __device__ inline int64_t oz_align256(int64_t n) { return (n + 255) & ~(int64_t)255; }
__host__ __device__ inline int64_t oz_f64_bytes(int64_t d) { return oz_align256(40 * d * d); }
struct OzLayout {
  int64_t plane;     // bytes per plane, dp * dp
  int n_slot4;       // persistent planes (M's 0..5, then T4's) in the fifth slot
  int n_half3;       // ... then in half-slot 3
  int t2_in_slot;    // T2's planes in the slot that will take M'
  int64_t extra;     // bytes past the float64 slots: exponents, then the other planes
};
__host__ __device__ inline OzLayout oz_layout(int64_t d) {
  OzLayout L;
  const int64_t dp = oz_pad(d), d2 = d * d;
  L.plane = dp * dp;
  const bool holes = d % 4 == 0;
  const int64_t b = holes ? 8 * d2 / L.plane : 0, a = holes ? 4 * d2 / L.plane : 0;
  L.n_slot4 = (int)(b < 2 * kOzSlices ? b : 2 * kOzSlices);
  L.n_half3 = (int)(a < 2 * kOzSlices - L.n_slot4 ? a : 2 * kOzSlices - L.n_slot4);
  L.t2_in_slot = holes && kOzSlices * L.plane <= 8 * d2 ? 1 : 0;
  const int64_t over = 2 * kOzSlices - L.n_slot4 - L.n_half3 + (L.t2_in_slot ? 0 : kOzSlices);
  L.extra = oz_align256(4 * dp) + over * L.plane;
  return L;
}

// Workgroup ranges of jobs and size classes start on multiples of 8 (one per
// XCD) and are padded to a multiple of 8.
__host__ __device__ inline int32_t round8(int32_t n) { return (n + 7) & ~7; }

// Per-matrix state of one inv_quarter_root_batched call (device, in the
// workspace).  Slot order: Newton matrices grouped by size class, then the
// Jacobi matrices.  64 bytes.
struct RootState {
  double s;          // rescale: trace(A) or 1
  double c;          // bound on lambda_max(A/s + eps I) (Newton)
  double out_scale;  // c^(-1/4)
  double eps;
  int32_t d;
  int32_t K;  // Newton iterations of this matrix
  int32_t j;  // first float32 iteration (== K when all float64)
  uint32_t flags;
  float residual;
  int32_t method;  // MR_JACOBI or MR_NEWTON
  int32_t sweeps;
  int32_t problem;  // index of the problem in the caller's array
  int32_t fin;      // degree in M of the last Newton step's X update (1, 2 or 4)
  int32_t pad;
};
static_assert(sizeof(RootState) == 72, "RootState layout");

// ---------------------------------------------------------------- Gram EMA
struct SyrkJob {
  const float* G;
  int64_t ldg;
  void* S;
  int64_t lds;
  int32_t d;            // Gram dimension (m left, n right)
  int32_t K;            // contraction length (n left, m right)
  int32_t T;            // tiles per side
  int32_t block_begin;  // first workgroup of this job (multiple of 8; range round8(T(T+1)/2))
};
static_assert(sizeof(SyrkJob) * kMaxSyrkJobs + 64 < 4096, "Gram EMA table fits the kernel arguments");
struct SyrkBatch {
  SyrkJob job[kMaxSyrkJobs];
  int32_t njobs;
  int32_t total_blocks;
  double alpha;  // 1 - beta
  double beta;
  int32_t packed;  // states stored packed (MR_PACKED)
  int32_t pad;
};

// Split-fp16 apply: operands are split copies of 2^s times a float32 matrix,
// s per matrix such that the largest magnitude lands in [2^14, 2^15) (so
// neither half overflows fp16 or loses precision to its subnormals, whatever
// the matrix's scale), rows padded to a multiple of 32 and zero-filled,
// written by split_pad_kernel; a split matrix of r rows and row stride ld is
// its hi half (r * ld fp16) followed by its lo half.  The largest magnitude
// of each matrix comes from absmax_kernel, as the bits of a float32 (for
// non-negative floats their order is that of the unsigned bit patterns, and a
// NaN sorts above infinity), combined with atomicMax over workgroups.
struct X3ApplyJob {
  const _Float16* a;     // split, M rows, row stride ld
  const _Float16* b;     // split, N rows, row stride ld
  float* c;              // float32 output, row stride ldc
  const uint32_t* a_max; // largest magnitude of A's float32 source (sets its scale)
  const uint32_t* b_max;
  int64_t ld;            // the padded contraction length K (a multiple of 32)
  int64_t ldc;
  int32_t M, N;
  int32_t tiles_n;
  int32_t block_begin;   // multiple of 8
  int32_t nblocks;
  float alpha;           // C = alpha * A * B^T of the unscaled matrices
};
constexpr int kMaxX3ApplyJobs = 48;
static_assert(sizeof(X3ApplyJob) * kMaxX3ApplyJobs + 64 < 4096, "split apply table fits the kernel arguments");
struct X3ApplyBatch {
  X3ApplyJob job[kMaxX3ApplyJobs];
  int32_t njobs;
  int32_t total_blocks;
};
// One float32 matrix times 2^s into split form at dst (rows x ldd, ldd >= cols
// a multiple of 8; columns cols .. ldd - 1 zero); s from the matrix's largest
// magnitude *amax.  trans = 0: dst row r is src row r (src rows x cols, row
// stride lds; 2048 elements per workgroup).  trans = 1: dst row r is src
// column r (src cols x rows; 64 x 64 dst tiles per workgroup, through LDS).
struct SplitPadJob {
  const float* src;
  _Float16* dst;
  const uint32_t* amax;
  int64_t lds, ldd;
  int32_t rows, cols;
  int32_t block_begin;  // first workgroup of this job
  int16_t vec4;         // src rows 16-byte aligned (float4 loads; trans = 0)
  int16_t trans;
};
// Largest magnitude of a float32 matrix into *amax (zeroed beforehand), a
// workgroup per kAbsMaxRows-row band.
constexpr int kAbsMaxRows = 16;
struct AbsMaxJob {
  const float* src;
  uint32_t* amax;
  int64_t lds;
  int32_t rows, cols;
  int32_t block_begin;
  int32_t vec4;  // rows 16-byte aligned, cols a multiple of 4
};
constexpr int kMaxAbsMaxJobs = 64;
struct AbsMaxBatch {
  AbsMaxJob job[kMaxAbsMaxJobs];
  int32_t njobs;
  int32_t total_blocks;
};
constexpr int kMaxSplitPadJobs = 64;
static_assert(sizeof(SplitPadJob) * kMaxSplitPadJobs + 64 < 4096, "split table fits the kernel arguments");
struct SplitPadBatch {
  SplitPadJob job[kMaxSplitPadJobs];
  int32_t njobs;
  int32_t total_blocks;
};

// ------------------------------------------------------ root: per-matrix
struct RootJob {
  const void* A;
  int64_t lda;
  float* X;
  int64_t ldx;
  char* region;  // Newton buffers (5 float64 slots of d*d, then the digit planes), NULL for Jacobi
  int32_t d;
  int32_t slot;     // index into the RootState array
  int32_t problem;  // index in the caller's problem array
  int32_t block_begin;
  int32_t nblocks;
  int32_t pad;
};
static_assert(sizeof(RootJob) * kMaxRootJobs + 128 < 4096, "root table fits the kernel arguments");
struct RootBatch {
  RootJob job[kMaxRootJobs];
  int32_t njobs;
  int32_t total_blocks;
  int32_t a_f64;      // A is float64
  int32_t normalize;  // MR_NORM_*
  double eps;
  RootState* state;
  double* partial;         // per-workgroup partial sums
  int64_t partial_stride;  // doubles per matrix slot in `partial`
  int32_t x_low;           // X kept in float32 from the first step
  int32_t a_packed;        // A stored packed (MR_PACKED)
  const double* sched;     // per-slot step scales (kMaxNewtonIters each)
};

// ------------------------------------------------ Newton: per size class
struct NewtonClass {
  char* region;          // buffers of the class's first matrix
  int64_t matrix_bytes;  // distance between consecutive matrices' buffers
  int32_t d, count, T, U;  // size, matrices, tiles per side, upper tiles
  int32_t block_begin;     // first workgroup of this class in the launch (multiple of 8)
  int32_t slot_begin;      // RootState slot of the class's first matrix
  int32_t blocks_per_matrix;
  int32_t nblocks;         // count * blocks_per_matrix (range is round8(nblocks) long)
};
struct NewtonLaunch {
  NewtonClass cls[kMaxClasses];
  int32_t ncls;
  int32_t total_blocks;
  int32_t stage;  // GEMM stages: 0 -> T2 and X', 1 -> T4, 2 -> M'
  int32_t t;      // iteration
  RootState* state;
  const double* sched;  // per slot: kMaxNewtonIters step scales
  int32_t x_low;        // X kept in float32 from the first step
  int32_t job_only;     // -1: every job of the stage; else only that job
  int32_t wide;         // split-fp16 stages on 256 x 256 tiles (every class's d a multiple of 32)
};

// ------------------------------------------------------------ Jacobi
// One matrix of a Jacobi launch; the host writes the batch's records into the
// workspace (jacobi_desc_kernel) and each launch reads its size class's range.
struct JacobiDesc {
  const void* A;
  int64_t lda;
  float* X;
  int64_t ldx;
  double* W;  // d*d float64 eigenvector scratch in the workspace (d > 96 only)
  int32_t d;
  int32_t slot;
  int32_t problem;
  int32_t pad;
};
static_assert(sizeof(JacobiDesc) == 56, "JacobiDesc layout");
constexpr int kMaxJacobiDesc = 64;
struct JacobiDescBatch {
  JacobiDesc desc[kMaxJacobiDesc];
  JacobiDesc* dst;  // the workspace table
  int32_t first, count;
};
static_assert(sizeof(JacobiDescBatch) + 64 < 4096, "Jacobi descriptor batch fits the kernel arguments");
// Jacobi size classes: padded size n = d + (d odd) <= kJacobiClass[k]; W in
// LDS for classes up to kJacobiLdsW.
constexpr int kJacobiClasses = 4;
constexpr int kJacobiClass[kJacobiClasses] = {32, 64, 96, 128};
constexpr int kJacobiLdsW = 96;
__host__ __device__ inline int jacobi_class_of(int64_t d) {
  const int64_t n = d + (d & 1);
  return n <= 32 ? 0 : n <= 64 ? 1 : n <= 96 ? 2 : 3;
}
struct JacobiLaunch {
  const JacobiDesc* desc;
  RootState* state;
  double eps;
  int32_t first;  // first record of this launch; one workgroup per record
  int32_t count;
  int32_t normalize;
  int32_t max_sweeps;
  int32_t a_packed;  // A stored packed (MR_PACKED)
  int32_t pad;
};

// ------------------------------------------------------------ launchers
// Each returns the HIP error of its launch (hipSuccess when launched).
hipError_t launch_syrk_ema(const SyrkBatch& b, bool right, bool f64_state, int vec, hipStream_t s);
hipError_t launch_split_pad(const SplitPadBatch& b, hipStream_t s);
hipError_t launch_split_pad_t(const SplitPadBatch& b, hipStream_t s);
hipError_t launch_absmax(const AbsMaxBatch& b, hipStream_t s);
hipError_t launch_fill_zero(uint32_t* p, int32_t n, hipStream_t s);
hipError_t launch_x3_apply(const X3ApplyBatch& b, hipStream_t s);

hipError_t launch_root_stats(const RootBatch& b, hipStream_t s);
hipError_t launch_root_bound(RootState* state, double* partial, int64_t partial_stride, double* sched,
                             int32_t slot_begin, int32_t nslots, int32_t normalize, double eps,
                             int32_t k_cap, double floor_cap, int32_t all_f64, int32_t finish, hipStream_t s);
hipError_t launch_root_init(const RootBatch& b, hipStream_t s);
// Moment bounds on the largest eigenvalue (Newton matrices with d >=
// kMomentMinD): fp16 copy H of (A/s + eps I)/c zero-padded to moment_pad(d),
// the tile sums of squares of H H (fourth moment) and of its fp16 copy
// squared (eighth moment) into the partials, then the tighter c and its
// schedule.
constexpr int kMomentMinD = 256;  // below, three more launches outweigh the steps a tighter bound saves
constexpr int kMomentTile = 128;
__host__ __device__ inline int moment_pad(int d) { return (d + 63) / 64 * 64; }
__host__ __device__ inline int moment_tiles(int d) {
  const int t = (moment_pad(d) + kMomentTile - 1) / kMomentTile;
  return t * (t + 1) / 2;
}
hipError_t launch_root_moment_convert(const RootBatch& b, hipStream_t s);
hipError_t launch_root_moment(const RootBatch& b, int pass, hipStream_t s);
hipError_t launch_root_tighten(RootState* state, const double* partial, int64_t partial_stride, double* sched,
                               int32_t slot_begin, int32_t nslots, double eps, int32_t k_cap, double floor_cap,
                               int32_t all_f64, int32_t finish, hipStream_t s);
enum StageKind { kStageF64 = 0, kStageF32 = 1, kStageX3 = 2, kStageX3B64 = 3, kStageI8 = 4 };
hipError_t launch_newton_stage(const NewtonLaunch& L, int kind, int vec, hipStream_t s);
hipError_t launch_newton_slice(const NewtonLaunch& L, hipStream_t s);
hipError_t launch_newton_convert(const NewtonLaunch& L, hipStream_t s);
hipError_t launch_root_finalize(const RootBatch& b, hipStream_t s);
hipError_t launch_root_info(RootState* state, const double* partial, int64_t partial_stride,
                            int32_t count, mr_root_info* info, hipStream_t s);
hipError_t launch_jacobi(const JacobiLaunch& L, int nmax, bool a_f64, hipStream_t s);
hipError_t launch_jacobi_desc(const JacobiDescBatch& b, hipStream_t s);

}  // namespace mr
