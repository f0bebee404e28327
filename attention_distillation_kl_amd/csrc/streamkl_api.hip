// streamkl_api.hip -- the C ABI declared in include/streamkl.h: argument
// validation, then dispatch to the forward / backward kernels.  No device
// memory is allocated here.  The only state kept between calls is the
// per-device address of the fixed scratch array of
// streamkl_fwd_splitk_noalloc, looked up on its first call on a device.
#include "streamkl.h"
#include "streamkl_launch.h"

#include <cmath>
#include <cstdint>
#include <mutex>

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

#ifdef STREAMKL_DEBUG
unsigned streamkl_debug_take(void) {
  const unsigned w[] = {streamkl::dbg_take_fwd(), streamkl::dbg_take_bwd_dk(), streamkl::dbg_take_bwd_dq(),
                        streamkl::dbg_take_bwd_fused()};
  for (unsigned x : w)
    if (x) return x;
  return 0;
}
#endif

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

bool split_args_ok(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  if (B <= 0 || H <= 0 || N_Q <= 0 || N_K <= 0 || (d != 64 && d != 128)) return false;
  if ((dtype != STREAMKL_F32 && dtype != STREAMKL_BF16) || grad_mask < 1 || grad_mask > 3) return false;
  return (long long)B * H <= INT32_MAX;
}

// Key partitions of the query-gradient kernel for these arguments (1 = none).
int bwd_dq_splits(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  if (!split_args_ok(B, H, N_Q, N_K, d, dtype, grad_mask)) return 1;
  return streamkl::bwd_dq_default_splits(B * H, N_Q, N_K, d, dtype == STREAMKL_BF16, grad_mask);
}

// Query partitions of the key-gradient kernel for these arguments (1 = none).
int bwd_dk_splits(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  if (!split_args_ok(B, H, N_Q, N_K, d, dtype, grad_mask)) return 1;
  return streamkl::bwd_dk_default_splits(B * H, N_Q, N_K, d, dtype == STREAMKL_BF16, grad_mask);
}

}  // namespace

namespace {

// Workspace of the query-gradient half with key partitions (0 without).
size_t dq_ws_bytes(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  const int s = bwd_dq_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
  if (s <= 1) return 0;
  return streamkl::bwd_dq_workspace_floats(B * H, N_Q, d, grad_mask, s) * sizeof(float);
}

// Workspace of the key-gradient half with query partitions (0 without).
size_t dk_ws_bytes(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  const int s = bwd_dk_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
  if (s <= 1) return 0;
  return streamkl::bwd_dk_workspace_floats(B * H, N_K, d, grad_mask, s) * sizeof(float);
}

// The two-kernel form's workspace: the halves run one after the other on one
// stream and share it.
size_t partitioned_ws_bytes(int B, int H, int N_Q, int N_K, int d, int dtype, int grad_mask) {
  const size_t q = dq_ws_bytes(B, H, N_Q, N_K, d, dtype, grad_mask);
  const size_t k = dk_ws_bytes(B, H, N_Q, N_K, d, dtype, grad_mask);
  return q > k ? q : k;
}

// Combined L2 of the eight XCDs (4 MiB each).
constexpr size_t kL2Bytes = size_t(32) << 20;

}  // namespace

int streamkl_bwd_fused_selected(int B, int H, int N_Q, int N_K, int d, int causal, int dtype, int grad_mask) {
  if (B <= 0 || H <= 0 || N_Q <= 0 || N_K <= 0 || (d != 64 && d != 128)) return 0;
  if (dtype != STREAMKL_BF16 || grad_mask < 1 || grad_mask > 3 || (long long)B * H > INT32_MAX) return 0;
  if (causal && N_Q > N_K) return 0;
  // Short query blocks only, where the fused form measured faster than the
  // two-kernel form: one 64-row query tile per head, which a workgroup keeps
  // while it walks its key blocks (1.2-2.5x at d = 128 and d = 64 from 8K
  // keys per head; 0.76-1.6x, calls of 30-60 us, on small grids of 2K-16K
  // keys; slower from 96 queries, with a second tile).  And the fp32
  // query-gradient buffer within L2, the page's criterion.
  if (N_Q > 64) return 0;
  return streamkl::bwd_fused_workspace_floats(B * H, N_Q, d, grad_mask) * sizeof(float) <= kL2Bytes ? 1 : 0;
}

size_t streamkl_bwd_workspace_size(int B, int H, int N_Q, int N_K, int d, int causal, int dtype,
                                   int grad_mask) {
  const size_t part = partitioned_ws_bytes(B, H, N_Q, N_K, d, dtype, grad_mask);
  if (!streamkl_bwd_fused_selected(B, H, N_Q, N_K, d, causal, dtype, grad_mask)) return part;
  const size_t fused = streamkl::bwd_fused_workspace_floats(B * H, N_Q, d, grad_mask) * sizeof(float);
  return fused > part ? fused : part;  // enough for streamkl_bwd_dq_ws as well
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

// Checks the caller's workspace against what the requested halves need (dq:
// the query-gradient kernel's key partitions, dk: the key-gradient kernel's
// query partitions) and switches each half that has partitions to them, with
// their partial sums in the workspace.
streamkl_status attach_workspace(streamkl::BwdArgs &a, int B, int H, int N_Q, int N_K, int d, int dtype,
                                 int grad_mask, void *workspace, size_t workspace_bytes, bool dq, bool dk) {
  const size_t nq = dq ? dq_ws_bytes(B, H, N_Q, N_K, d, dtype, grad_mask) : 0;
  const size_t nk = dk ? dk_ws_bytes(B, H, N_Q, N_K, d, dtype, grad_mask) : 0;
  const size_t need = nq > nk ? nq : nk;
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return STREAMKL_ERR_WORKSPACE;
  if (need > 0) a.part = static_cast<float *>(workspace);
  if (nq > 0) a.dq_splits = bwd_dq_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
  if (nk > 0) a.dk_splits = bwd_dk_splits(B, H, N_Q, N_K, d, dtype, grad_mask);
  return STREAMKL_OK;
}

}  // namespace

streamkl_status streamkl_bwd(const void *q1, const void *k1, const void *q2, const void *k2,
                             const float *kl, const float *lse1, const float *lse2, const float *dkl,
                             int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                             int grad_mask, void *dq1, void *dk1, void *dq2, void *dk2, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (streamkl_bwd_fused_selected(B, H, N_Q, N_K, d, causal, dtype, grad_mask))
    return streamkl_bwd_fused(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal, dtype,
                              grad_mask, dq1, dk1, dq2, dk2, workspace, workspace_bytes, stream);
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, dq1, dk1, dq2, dk2, true, true, a);
  if (s != STREAMKL_OK) return s;
  s = attach_workspace(a, B, H, N_Q, N_K, d, dtype, grad_mask, workspace, workspace_bytes, true, true);
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
  s = attach_workspace(a, B, H, N_Q, N_K, d, dtype, grad_mask, workspace, workspace_bytes, true, false);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_dq(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                     : STREAMKL_ERR_HIP;
}

streamkl_status streamkl_bwd_dk_ws(const void *q1, const void *k1, const void *q2, const void *k2,
                                   const float *kl, const float *lse1, const float *lse2, const float *dkl,
                                   int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                   int grad_mask, void *dk1, void *dk2, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, nullptr, dk1, nullptr, dk2, false, true, a);
  if (s != STREAMKL_OK) return s;
  s = attach_workspace(a, B, H, N_Q, N_K, d, dtype, grad_mask, workspace, workspace_bytes, false, true);
  if (s != STREAMKL_OK) return s;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_dk(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
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

size_t streamkl_bwd_fused_workspace_size(int B, int H, int N_Q, int N_K, int d, int causal, int dtype,
                                         int grad_mask) {
  (void)N_K, (void)causal;
  if (B <= 0 || H <= 0 || N_Q <= 0 || (d != 64 && d != 128) || dtype != STREAMKL_BF16) return 0;
  if (grad_mask < 1 || grad_mask > 3 || (long long)B * H > INT32_MAX) return 0;
  return streamkl::bwd_fused_workspace_floats(B * H, N_Q, d, grad_mask) * sizeof(float);
}

streamkl_status streamkl_bwd_fused(const void *q1, const void *k1, const void *q2, const void *k2,
                                   const float *kl, const float *lse1, const float *lse2, const float *dkl,
                                   int B, int H, int N_Q, int N_K, int d, float scale, int causal, int dtype,
                                   int grad_mask, void *dq1, void *dk1, void *dq2, void *dk2, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  streamkl::BwdArgs a;
  streamkl_status s = prepare_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl, B, H, N_Q, N_K, d, scale, causal,
                                  dtype, grad_mask, dq1, dk1, dq2, dk2, true, true, a);
  if (s != STREAMKL_OK) return s;
  if (dtype != STREAMKL_BF16) return STREAMKL_ERR_UNSUPPORTED;
  const size_t need = streamkl_bwd_fused_workspace_size(B, H, N_Q, N_K, d, causal, dtype, grad_mask);
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return STREAMKL_ERR_WORKSPACE;
  if (bwd_is_noop(B, H, N_Q, N_K)) return STREAMKL_OK;
  return streamkl::launch_bwd_fused(a, static_cast<float *>(workspace), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? STREAMKL_OK
             : STREAMKL_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- no-alloc
// Partition states of streamkl_fwd_splitk_noalloc: a fixed array in device
// memory, one copy per GPU, alive until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to a kernel.
static __device__ __align__(256) float scratch[STREAMKL_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device

// Device address of `scratch` on the calling thread's current device, or
// nullptr if the runtime cannot tell the device or resolve the symbol.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" streamkl_status streamkl_fwd_splitk_noalloc(const void *q1, const void *k1, const void *q2,
                                                       const void *k2, int B, int H, int N_Q, int N_K, int d,
                                                       float scale, int causal, int dtype, int splits, float *kl,
                                                       float *lse1, float *lse2, void *stream) {
  streamkl_status s = check_common(q1, k1, q2, k2, B, H, N_Q, N_K, d, scale, causal, dtype);
  if (s != STREAMKL_OK) return s;
  if (splits < 1 || splits > STREAMKL_MAX_SPLITS) return STREAMKL_ERR_INVALID_ARGUMENT;
  const long long rows = (long long)B * H * N_Q;
  if (!row_vec_ok(kl, rows) || !row_vec_ok(lse1, rows) || !row_vec_ok(lse2, rows))
    return STREAMKL_ERR_INVALID_ARGUMENT;
  const size_t need = streamkl_fwd_workspace_size(B, H, N_Q, N_K, d, causal, dtype, splits);
  if (need > STREAMKL_NOALLOC_SCRATCH_BYTES) return STREAMKL_ERR_WORKSPACE;
  if (rows == 0) return STREAMKL_OK;
  streamkl::FwdArgs a{q1, k1, q2, k2, kl, lse1, lse2, B * H, N_Q, N_K, d, scale, causal != 0,
                      dtype == STREAMKL_BF16};
  a.splits = splits;
  if (splits > 1) {
    // Every (partition, row) state the merge reads is written by the split
    // kernel of the same call, so nothing needs clearing first.
    a.part = static_cast<float *>(scratch_on_current_device());
    if (!a.part) return STREAMKL_ERR_HIP;
  }
  return streamkl::launch_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? STREAMKL_OK
                                                                                  : STREAMKL_ERR_HIP;
}
