// streamkl_launch.h -- internal interface between the C ABI layer and the
// kernel translation units.  Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace streamkl {

struct FwdArgs {
  const void *q1, *k1, *q2, *k2;
  float *kl, *lse1, *lse2;
  int bh, nq, nk, d;
  float scale;
  bool causal, bf16;
  int splits = 1;           // key partitions (split-K) when > 1
  float *part = nullptr;    // their row states: 5 * splits * bh * nq floats
};

struct BwdArgs {
  const void *q1, *k1, *q2, *k2;
  const float *kl, *lse1, *lse2, *dkl;
  void *dq1, *dk1, *dq2, *dk2;
  int bh, nq, nk, d;
  float scale;
  bool causal, bf16;
  int grad_mask;  // 1: dq1/dk1, 2: dq2/dk2, 3: both
  int dq_splits = 1;       // key partitions of the query-gradient kernel when > 1
  float *part = nullptr;   // their fp32 partial gradients (see bwd_dq_workspace_floats)
};

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
// The library's choice of key partitions for a forward problem (1 = none).
int fwd_default_splits(int bh, int nq, int nk, int d, bool bf16, bool causal);
// The library's choice of key partitions for the query-gradient kernel, and
// the fp32 workspace it then needs (splits * bh * nq * d per requested
// gradient; 0 when splits == 1).
int bwd_dq_default_splits(int bh, int nq, int nk, int d, bool bf16, int grad_mask);
size_t bwd_dq_workspace_floats(int bh, int nq, int d, int grad_mask, int splits);
hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t stream);
hipError_t launch_bwd_dk(const BwdArgs &a, hipStream_t stream);

}  // namespace streamkl
