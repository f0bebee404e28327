// streamkl_api.hip -- the C ABI declared in include/streamkl.h: argument
// validation, then dispatch to the forward / backward kernels.  No device
// memory is allocated here and no state is kept between calls.
#include "streamkl.h"
#include "streamkl_launch.h"

#include <cmath>
#include <cstdint>

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks common to both passes.  Returns STREAMKL_OK or the error to report.
streamkl_status check_common(const void *q1, const void *k1, const void *q2, const void *k2, int B,
                             int H, int N_Q, int N_K, int d, float scale, int causal, int dtype) {
  if (B < 0 || H < 0 || N_Q < 0 || N_K < 0 || d < 0) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale) || !(scale > 0.f)) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (causal != 0 && causal != 1) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) return STREAMKL_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return STREAMKL_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  if (bh > INT32_MAX) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (bh == 0) return STREAMKL_OK;
  if (N_Q > 0 && N_K == 0) return STREAMKL_ERR_INVALID_ARGUMENT;  // rows with no keys
  if (causal && N_Q > N_K) return STREAMKL_ERR_INVALID_ARGUMENT;  // rows with no keys
  if (N_Q > 0 && (!q1 || !q2 || !aligned16(q1) || !aligned16(q2))) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (N_K > 0 && (!k1 || !k2 || !aligned16(k1) || !aligned16(k2))) return STREAMKL_ERR_INVALID_ARGUMENT;
  return STREAMKL_OK;
}

bool row_vec_ok(const void *p, long long n) { return n == 0 || (p && aligned16(p)); }

}  // namespace

extern "C" {

const char *streamkl_status_str(int status) {
  switch (status) {
    case STREAMKL_OK: return "STREAMKL_OK";
    case STREAMKL_ERR_INVALID_ARGUMENT: return "STREAMKL_ERR_INVALID_ARGUMENT";
    case STREAMKL_ERR_UNSUPPORTED: return "STREAMKL_ERR_UNSUPPORTED";
    case STREAMKL_ERR_WORKSPACE: return "STREAMKL_ERR_WORKSPACE";
    case STREAMKL_ERR_HIP: return "STREAMKL_ERR_HIP";
    default: return "STREAMKL_ERR_UNKNOWN";
  }
}

int streamkl_abi_version(void) { return 1; }

streamkl_status streamkl_fwd(const void *q1, const void *k1, const void *q2, const void *k2, int B, int H,
                             int N_Q, int N_K, int d, float scale, int causal, int dtype, float *kl,
                             float *lse1, float *lse2, void *stream) {
  streamkl_status s = check_common(q1, k1, q2, k2, B, H, N_Q, N_K, d, scale, causal, dtype);
  if (s != STREAMKL_OK) return s;
  const long long rows = (long long)B * H * N_Q;
  if (!row_vec_ok(kl, rows) || !row_vec_ok(lse1, rows) || !row_vec_ok(lse2, rows))
    return STREAMKL_ERR_INVALID_ARGUMENT;
  if (rows == 0) return STREAMKL_OK;
  streamkl::FwdArgs a{q1, k1, q2, k2, kl, lse1, lse2, B * H, N_Q, N_K, d, scale, causal != 0,
                      dtype == STREAMKL_BF16};
  return streamkl::launch_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                  : STREAMKL_ERR_HIP;
}

int streamkl_fwd_splits(int B, int H, int N_Q, int N_K, int d, int causal, int dtype) {
  if (B <= 0 || H <= 0 || N_Q <= 0 || N_K <= 0 || (d != 64 && d != 128)) return 1;
  if (dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) return 1;
  const long long bh = (long long)B * H;
  if (bh > INT32_MAX) return 1;
  return streamkl::fwd_default_splits(int(bh), N_Q, N_K, d, dtype == STREAMKL_BF16, causal != 0);
}

size_t streamkl_fwd_workspace_size(int B, int H, int N_Q, int N_K, int d, int causal, int dtype, int splits) {
  (void)N_K, (void)d, (void)causal, (void)dtype;
  if (splits <= 1 || B <= 0 || H <= 0 || N_Q <= 0) return 0;
  return size_t(5) * size_t(splits) * size_t(B) * size_t(H) * size_t(N_Q) * sizeof(float);
}

streamkl_status streamkl_fwd_splitk(const void *q1, const void *k1, const void *q2, const void *k2, int B,
                                    int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                    int splits, float *kl, float *lse1, float *lse2, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  streamkl_status s = check_common(q1, k1, q2, k2, B, H, N_Q, N_K, d, scale, causal, dtype);
  if (s != STREAMKL_OK) return s;
  if (splits < 1 || splits > STREAMKL_MAX_SPLITS) return STREAMKL_ERR_INVALID_ARGUMENT;
  const long long rows = (long long)B * H * N_Q;
  if (!row_vec_ok(kl, rows) || !row_vec_ok(lse1, rows) || !row_vec_ok(lse2, rows))
    return STREAMKL_ERR_INVALID_ARGUMENT;
  const size_t need = streamkl_fwd_workspace_size(B, H, N_Q, N_K, d, causal, dtype, splits);
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace))))
    return STREAMKL_ERR_WORKSPACE;
  if (rows == 0) return STREAMKL_OK;
  streamkl::FwdArgs a{q1, k1, q2, k2, kl, lse1, lse2, B * H, N_Q, N_K, d, scale, causal != 0,
                      dtype == STREAMKL_BF16};
  a.splits = splits;
  a.part = static_cast<float *>(workspace);
  return streamkl::launch_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                  : STREAMKL_ERR_HIP;
}

namespace {

// Key partitions of the query-gradient kernel for these arguments (1 = none).
int bwd_dq_splits(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  if (B <= 0 || H <= 0 || N_Q <= 0 || N_K <= 0 || (d != 64 && d != 128)) return 1;
  if ((dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) || grad_mask < 1 || grad_mask > 3) return 1;
  const long long bh = (long long)B * H;
  if (bh > INT32_MAX) return 1;
  return streamkl::bwd_dq_default_splits(int(bh), N_Q, N_K, d, dtype == STREAMKL_BF16, grad_mask);
}

}  // namespace

size_t streamkl_bwd_workspace_size(int B, int H, int N_Q, int N_K, int d, int causal, int dtype,
                                   int grad_mask) {
  (void)causal;
  const int s = bwd_dq_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
  if (s <= 1) return 0;
  return streamkl::bwd_dq_workspace_floats(B * H, N_Q, d, grad_mask, s) * sizeof(float);
}

namespace {

// Validation shared by the backward entry points; fills `a` on success.
// need_q / need_k: whether the query / key gradient outputs are produced.
streamkl_status prepare_bwd(const void *q1, const void *k1, const void *q2, const void *k2,
                            const float *kl, const float *lse1, const float *lse2, const float *dkl,
                            int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                            int grad_mask, void *dq1, void *dk1, void *dq2, void *dk2, bool need_q,
                            bool need_k, streamkl::BwdArgs &a) {
  streamkl_status s = check_common(q1, k1, q2, k2, B, H, N_Q, N_K, d, scale, causal, dtype);
  if (s != STREAMKL_OK) return s;
  if (grad_mask < 1 || grad_mask > 3) return STREAMKL_ERR_INVALID_ARGUMENT;
  const long long bh = (long long)B * H;
  const long long rows = bh * N_Q, kn = bh * N_K;
  const bool g1 = grad_mask & 1, g2 = grad_mask & 2;
  if (!row_vec_ok(kl, rows) || !row_vec_ok(lse1, rows) || !row_vec_ok(lse2, rows))
    return STREAMKL_ERR_INVALID_ARGUMENT;
  if (dkl && !aligned16(dkl)) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (need_q && g1 && !row_vec_ok(dq1, rows)) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (need_q && g2 && !row_vec_ok(dq2, rows)) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (need_k && g1 && !row_vec_ok(dk1, kn)) return STREAMKL_ERR_INVALID_ARGUMENT;
  if (need_k && g2 && !row_vec_ok(dk2, kn)) return STREAMKL_ERR_INVALID_ARGUMENT;
  a = streamkl::BwdArgs{q1, k1, q2, k2, kl, lse1, lse2, dkl, dq1, dk1, dq2, dk2, int(bh), N_Q, N_K, d,
                        scale, causal != 0, dtype == STREAMKL_BF16, grad_mask};
  return STREAMKL_OK;
}

bool bwd_is_noop(int B, int H, int N_Q, int N_K) { return (long long)B * H == 0 || (N_Q == 0 && N_K == 0); }

// Checks the caller's workspace against streamkl_bwd_workspace_size and, where
// that size is not zero (short query blocks), switches the query-gradient
// kernel to key partitions whose partial sums go to the workspace.
streamkl_status attach_dq_workspace(streamkl::BwdArgs &a, int B, int H, int N_Q, int N_K, int d, int causal,
                                    int dtype, int grad_mask, void *workspace, size_t workspace_bytes) {
  const size_t need = streamkl_bwd_workspace_size(B, H, N_Q, N_K, d, causal, dtype, grad_mask);
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return STREAMKL_ERR_WORKSPACE;
  if (need > 0) {
    a.dq_splits = bwd_dq_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
    a.part = static_cast<float *>(workspace);
  }
  return STREAMKL_OK;
}

}  // namespace

streamkl_status streamkl_bwd(const void *q1, const void *k1, const void *q2, const void *k2,
                             const float *kl, const float *lse1, const float *lse2, const float *dkl,
                             int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                             int grad_mask, void *dq1, void *dk1, void *dq2, void *dk2, void *workspace,
                             size_t workspace_bytes, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, dq1, dk1, dq2, dk2, true, true, a);
  if (s != STREAMKL_OK) return s;
  s = attach_dq_workspace(a, B, H, N_Q, N_K, d, causal, dtype, grad_mask, workspace, workspace_bytes);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // The key-gradient kernel also runs when N_Q == 0: it then writes zeros.
  if (streamkl::launch_bwd_dk(a, st) != hipSuccess) return STREAMKL_ERR_HIP;
  if (streamkl::launch_bwd_dq(a, st) != hipSuccess) return STREAMKL_ERR_HIP;
  return STREAMKL_OK;
}

streamkl_status streamkl_bwd_dq(const void *q1, const void *k1, const void *q2, const void *k2,
                                const float *kl, const float *lse1, const float *lse2, const float *dkl,
                                int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                int grad_mask, void *dq1, void *dq2, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, dq1, nullptr, dq2, nullptr, true, false, a);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_dq(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                     : STREAMKL_ERR_HIP;
}

streamkl_status streamkl_bwd_dq_ws(const void *q1, const void *k1, const void *q2, const void *k2,
                                   const float *kl, const float *lse1, const float *lse2, const float *dkl,
                                   int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                   int grad_mask, void *dq1, void *dq2, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, dq1, nullptr, dq2, nullptr, true, false, a);
  if (s != STREAMKL_OK) return s;
  s = attach_dq_workspace(a, B, H, N_Q, N_K, d, causal, dtype, grad_mask, workspace, workspace_bytes);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_dq(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                     : STREAMKL_ERR_HIP;
}

streamkl_status streamkl_bwd_dk(const void *q1, const void *k1, const void *q2, const void *k2,
                                const float *kl, const float *lse1, const float *lse2, const float *dkl,
                                int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                int grad_mask, void *dk1, void *dk2, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, nullptr, dk1, nullptr, dk2, false, true, a);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_dk(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                     : STREAMKL_ERR_HIP;
}

}  // extern "C"
