// Host-side internals shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mssm.h"

namespace mssm {

// How one scan call is cut along time.  The sequence is split into K chunks
// of chunk_len steps (the last may be shorter).  Chunks 0..K-2 first produce
// summaries (their local end state from a zero start, and their decay
// exp(A * total step size)); each chunk then folds the summaries before it
// into its carry-in with the affine-pair operator and scans its own steps from
// that carry.
struct ScanPlan {
  int cpl = 1;                // chains (adjacent channels) per lane: 1 or 2
  int K = 1;
  int64_t chunk_len = 0;
  size_t sum_h_bytes = 0;     // float [batch][K-1][N][D]: chunk end state from zero
  size_t sum_p_offset = 0;    // byte offset of float [batch][K-1][N][D]: chunk decay
  size_t workspace_bytes = 0;
};



struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  void* y;
  int64_t batch, L, D, N;
  mssm_dtype dtype;
};

// Plan for `cpl` chains per lane.
ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, int cpl);

// Workspace that covers the plan of every chains-per-lane choice the launcher
// can make for this shape (the choice also depends on pointer alignment).
size_t workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N);

// Chains per lane for these arguments: 2 for bfloat16 inputs when D is even
// and x, delta, y are aligned for paired access, else 1.
int choose_cpl(const ScanArgs& a);

// Enqueues the scan kernels on `stream`.  Arguments are already validated and
// the workspace holds at least plan.workspace_bytes.  Returns hipSuccess or
// the launch error.
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& plan, void* workspace,
                       hipStream_t stream);

bool state_size_supported(int64_t N);

}  // namespace mssm
