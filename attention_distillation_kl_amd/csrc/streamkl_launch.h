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
  int dk_splits = 1;       // query partitions of the key-gradient kernel when > 1
  // The partitions' fp32 partial gradients (bwd_dq_workspace_floats,
  // bwd_dk_workspace_floats).  The key-gradient kernel and its reduction run
  // before the query-gradient kernel on the same stream, so the two roles
  // can share one workspace.
  float *part = nullptr;
};

// Whether a causal grid of nwg workgroups, nblk a head, takes its blocks
// longest first over each XCD's heads (longest_first in streamkl_device.h):
// where a head has fewer blocks than an XCD holds resident workgroups --
// only then does taking the heads one after the other leave long blocks for
// the end of the grid -- and each XCD's share of the grid is whole heads.
// Elsewhere that order only spreads more heads over each XCD's L2.
inline bool longest_first_pays(long long nwg, long long nblk, long long resident_per_xcd) {
  const long long per = nwg / 8;
  return nblk < resident_per_xcd && per > 0 && per % nblk == 0;
}

// Whether a causal grid takes the rank-major order (rank_major in
// streamkl_device.h) instead: more than one round of workgroups, and XCD
// shares that are not whole heads, so that head by head one XCD would get a
// head's long blocks and another its short ones.
inline bool rank_major_pays(long long nwg, long long nblk, long long resident_per_xcd) {
  const long long per = nwg / 8;
  return nwg > 8 * resident_per_xcd && nblk > 0 && (nwg % 8 != 0 || per % nblk != 0);
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);
// The library's choice of key partitions for a forward problem (1 = none).
int fwd_default_splits(int bh, int nq, int nk, int d, bool bf16, bool causal);
// The library's choice of key partitions for the query-gradient kernel, and
// the fp32 workspace it then needs (splits * bh * nq * d per requested
// gradient; 0 when splits == 1).
int bwd_dq_default_splits(int bh, int nq, int nk, int d, bool bf16, int grad_mask);
size_t bwd_dq_workspace_floats(int bh, int nq, int d, int grad_mask, int splits);
hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t stream);
// The same for the key-gradient kernel's query partitions (splits * bh * nk
// * d floats per requested gradient).
int bwd_dk_default_splits(int bh, int nq, int nk, int d, bool bf16, int grad_mask);
size_t bwd_dk_workspace_floats(int bh, int nk, int d, int grad_mask, int splits);
hipError_t launch_bwd_dk(const BwdArgs &a, hipStream_t stream);
// The single-pass backward (bf16 only): dK in registers, dQ added with
// atomics into `ws` (fp32, bwd_fused_workspace_floats values: the query
// gradients asked for, one after the other), then converted into dq1 / dq2.
size_t bwd_fused_workspace_floats(int bh, int nq, int d, int grad_mask);
hipError_t launch_bwd_fused(const BwdArgs &a, float *ws, hipStream_t stream);

#ifdef STREAMKL_DEBUG
// Debug builds: the first out-of-range access recorded by each translation
// unit's kernels since the last call (0: none), then cleared.
unsigned dbg_take_fwd();
unsigned dbg_take_bwd_dk();
unsigned dbg_take_bwd_dq();
unsigned dbg_take_bwd_fused();
#endif

}  // namespace streamkl
