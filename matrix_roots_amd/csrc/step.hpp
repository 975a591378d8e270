// Streaming kernels around the preconditioner (momentum EMA, hyperball
// update): launch descriptors shared by the host runtime and step.hip.
#pragma once

#include "launch.hpp"

namespace mr {

// One m x n float32 matrix pair: `inout` is updated in place (M for the
// momentum, W for the hyperball update), `in` is read (G, U).
struct StreamJob {
  const float* in;
  int64_t ld_in;
  float* inout;
  int64_t ld_inout;
  int32_t m, n;
  int32_t rows_per_block;
  int32_t block_begin, nblocks;  // this job's workgroups
  int32_t slot;                  // partial-sum slot (hyperball)
  int32_t problem;               // index in the caller's problem array
  int32_t pad;
};
// Up to 48 jobs per launch (2.7 KB of kernel arguments): a whole
// transformer block stack's weights in one HBM-bound pass instead of several
// short launches that each pay the ramp-up and tail.
constexpr int kMaxStreamJobs = 48;
struct StreamBatch {
  StreamJob job[kMaxStreamJobs];
  double* partial;  // hyperball: 3 doubles per workgroup, partial_stride per slot
  int64_t partial_stride;
  int32_t njobs, total_blocks;
};

// Rows per workgroup: about 8192 elements each, at least one row.
inline int32_t stream_rows_per_block(int64_t m, int64_t n) {
  int64_t r = 8192 / (n > 0 ? n : 1);
  if (r < 1) r = 1;
  if (r > m) r = m;
  return (int32_t)r;
}

hipError_t launch_momentum(const StreamBatch& b, int vec, double mu, hipStream_t s);
hipError_t launch_hyperball_reduce(const StreamBatch& b, int vec, hipStream_t s);
hipError_t launch_hyperball_update(const StreamBatch& b, int vec, double lr, double* norms, hipStream_t s);

}  // namespace mr
