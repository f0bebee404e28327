/*
 * streamkl.h -- C ABI of libstreamkl: fused attention-KL divergence between a
 * teacher and a student attention distribution, forward and recompute
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * The method is StreamKL as summarised on gist.science (paper 2606.20005):
 * for each query row i of each attention head,
 *
 *   S_t = scale * Q_t K_t^T        (t = 1 teacher, t = 2 student)
 *   P_t = softmax(S_t) over the allowed keys of the row
 *   KL[i] = KL(P1[i,:] || P2[i,:])
 *
 * computed in one pass over key tiles with five running row scalars
 * (two running shifts -- the page's running maxima, kept at or below them --,
 * two running exponential sums and one accumulator of the P1-weighted logit
 * difference), finalised as KL = acc/l1 + LSE2 - LSE1 with
 * LSE_t = m_t + log l_t ("Formulazione Online", forward pass section).
 * The N_Q x N_K matrices P1, P2 are never written to memory.  The backward
 * pass keeps only KL, LSE1 and LSE2 per row and regenerates
 * P_t = exp(S_t - LSE_t) tile by tile ("Strategia di Ricalcolo", backward
 * pass section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout    q1, q2: [B, H, N_Q, d]; k1, k2: [B, H, N_K, d]; contiguous, d
 *            innermost.  Row vectors kl, lse1, lse2, dkl: [B, H, N_Q] float32.
 *            Gradients have the shape and element type of the tensor they
 *            differentiate.
 *  Element   STREAMKL_BF16 (bfloat16 storage; products accumulate in fp32) or
 *  types     STREAMKL_F32.  KL and LSE are always float32.
 *  Logits    natural-log units of the scaled scores: LSE_t = log sum_j
 *            exp(scale * <q_t[i], k_t[j]>).  One scale for both
 *            distributions (fold a teacher temperature into q1).
 *  Causal    key j is allowed for query i iff j <= i + (N_K - N_Q), i.e. the
 *            mask is aligned to the bottom-right corner (j <= i when
 *            N_Q == N_K).  Requires N_Q <= N_K so every row has a key.
 *  Pointers  every tensor pointer is a DEVICE pointer owned by the caller and
 *            must be 16-byte aligned.  The library never allocates or frees
 *            device memory; apart from the fixed scratch array of
 *            streamkl_fwd_splitk_noalloc (and the cached per-device address
 *            of it) it keeps none and holds no global mutable state.  Outputs
 *            are fully overwritten and must not alias inputs.
 *  Streams   `stream` is a hipStream_t (NULL = the default stream).  Work is
 *            enqueued asynchronously; nothing synchronises the host.
 *  Errors    argument errors are reported before anything is enqueued; a
 *            failed launch (or no usable GPU) returns STREAMKL_ERR_HIP.
 *            Non-finite input values are not checked; they propagate.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STREAMKL_OK = 0,
  STREAMKL_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, scale, mask, ... */
  STREAMKL_ERR_UNSUPPORTED = 2,      /* d not in {64, 128} or unknown dtype */
  STREAMKL_ERR_WORKSPACE = 3,        /* workspace smaller than required     */
  STREAMKL_ERR_HIP = 4               /* HIP runtime / launch failure         */
} streamkl_status;

typedef enum { STREAMKL_F32 = 0, STREAMKL_BF16 = 1 } streamkl_dtype;

/* Which gradients the backward pass produces (the page's two
 * configurations; the two sets are independent partial derivatives). */
enum {
  STREAMKL_GRAD_Q1K1 = 1, /* Configuration 2: P2 held fixed, train P1 -> dq1, dk1 */
  STREAMKL_GRAD_Q2K2 = 2, /* Configuration 1: P1 held fixed, train P2 -> dq2, dk2 */
  STREAMKL_GRAD_ALL = 3
};

/*
 * streamkl_fwd -- forward pass ("Formulazione Online", forward pass section).
 *   in : q1, k1, q2, k2 (dtype), sizes B, H, N_Q, N_K, d, scale (> 0, finite),
 *        causal (0/1).
 *   out: kl[B,H,N_Q]   = KL(P1 || P2) per row (not clamped at 0),
 *        lse1, lse2    = log-sum-exp of the scaled teacher / student logits.
 * Causal key tiles beyond a query block's frontier are skipped, not masked.
 * B*H*N_Q == 0 is a valid no-op.
 */
streamkl_status streamkl_fwd(const void *q1, const void *k1, const void *q2,
                             const void *k2, int B, int H, int N_Q, int N_K,
                             int d, float scale, int causal, int dtype,
                             float *kl, float *lse1, float *lse2, void *stream);

/* Largest key-partition count streamkl_fwd_splitk accepts. */
#define STREAMKL_MAX_SPLITS 1024

/*
 * streamkl_fwd_splits -- the library's choice of key partitions for
 * streamkl_fwd_splitk on this problem: enough that short query blocks (few
 * workgroups per head, e.g. N_Q = 1 decoding or 2K queries over 64K keys)
 * still fill every compute unit once, at least four key tiles per
 * partition, and 1 (no split) when the unsplit grid already fills the GPU.
 * Causal problems with N_Q > N_K / 2, whose query blocks carry very
 * different amounts of work, get about four times as many workgroups (at
 * least 16 key tiles per partition) so that they balance -- unless the
 * unsplit grid spans more than one round of resident workgroups and the
 * kernel can take its query blocks longest first over each XCD's heads,
 * which balances it without partitions.  Invalid sizes give 1.
 */
int streamkl_fwd_splits(int B, int H, int N_Q, int N_K, int d, int causal, int dtype);

/*
 * streamkl_fwd_workspace_size -- bytes of device workspace streamkl_fwd_splitk
 * needs for `splits` partitions: 5 * splits * B * H * N_Q floats (the five
 * running row scalars of every partition), 0 when splits <= 1.
 */
size_t streamkl_fwd_workspace_size(int B, int H, int N_Q, int N_K, int d,
                                   int causal, int dtype, int splits);

/*
 * streamkl_fwd_splitk -- streamkl_fwd with the key dimension partitioned over
 * `splits` workgroups per query block ("Ottimizzazioni del Kernel GPU",
 * Split-K bullet: for small query counts the keys are partitioned across
 * thread blocks to fill the machine).  Partition s folds key tiles
 * [s*T, (s+1)*T), T = ceil(ceil(N_K / tile) / splits) (causal grids of more
 * than one round of workgroups: T = ceil(t / splits), t the query block's
 * own admissible tiles), into the five running scalars of each row and
 * stores them in `workspace`; a second kernel merges
 * the partitions with the same rescale as the online update
 * (m = max m_s, l = sum l_s exp(m_s - m), acc = sum acc_s exp(m1_s - m1)) and
 * finalises kl, lse1, lse2.  Results equal streamkl_fwd's up to the order of
 * floating-point summation; with splits == 1 they are identical.
 *   splits: 1 .. STREAMKL_MAX_SPLITS (see streamkl_fwd_splits).
 *   workspace / workspace_bytes: device memory of at least
 *        streamkl_fwd_workspace_size(...) bytes, 16-byte aligned (may be NULL
 *        when that is 0), owned by the caller, overwritten; its contents are
 *        dead once the call's work has completed on `stream`.
 * Errors as streamkl_fwd, plus STREAMKL_ERR_INVALID_ARGUMENT for a split
 * count out of range and STREAMKL_ERR_WORKSPACE for a missing, misaligned
 * or short workspace.
 */
streamkl_status streamkl_fwd_splitk(const void *q1, const void *k1,
                                    const void *q2, const void *k2, int B,
                                    int H, int N_Q, int N_K, int d,
                                    float scale, int causal, int dtype,
                                    int splits, float *kl, float *lse1,
                                    float *lse2, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Size of the fixed device scratch array of streamkl_fwd_splitk_noalloc. */
#define STREAMKL_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * streamkl_fwd_splitk_noalloc -- streamkl_fwd_splitk for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * (e.g. decoding rows over long key sets), harnesses that forbid hipMalloc.
 * It takes no workspace and allocates nothing: the partition states live in
 * a fixed array of STREAMKL_NOALLOC_SCRATCH_BYTES in device memory, one copy
 * per GPU, created when the library's code is loaded on that GPU and held
 * until the process ends.  The array is the one of the calling thread's
 * current device, which must be the device of `stream` and of the tensors;
 * its address is looked up on the first call on each device.
 *   Arguments, results and errors as streamkl_fwd_splitk (bitwise the same
 *   results for the same `splits`), without workspace / workspace_bytes.
 *   STREAMKL_ERR_WORKSPACE when streamkl_fwd_workspace_size(...) for these
 *   arguments exceeds STREAMKL_NOALLOC_SCRATCH_BYTES (5 * splits * B*H*N_Q
 *   floats must fit: e.g. 32 heads of 2048 queries at 16 partitions); a
 *   failed address lookup returns STREAMKL_ERR_HIP.
 * Every call on one GPU uses that GPU's one array, and a call leaves its
 * partition states there.  Calls on one GPU whose work may overlap (two
 * streams, or two host threads) race on it and give wrong results: order
 * them on one stream or with events.  Nothing needs clearing between calls:
 * each call writes every state it reads.
 */
streamkl_status streamkl_fwd_splitk_noalloc(const void *q1, const void *k1,
                                            const void *q2, const void *k2,
                                            int B, int H, int N_Q, int N_K,
                                            int d, float scale, int causal,
                                            int dtype, int splits, float *kl,
                                            float *lse1, float *lse2,
                                            void *stream);

/*
 * streamkl_bwd_workspace_size -- bytes of device workspace streamkl_bwd needs
 * for these arguments.  0 whenever the query-gradient and key-gradient grids
 * already fill the GPU.  For short query blocks (few query-row workgroups
 * per head) the query gradients are computed by key partitions, like the
 * split-K forward: each (query block, partition) workgroup stores its fp32
 * partial dq_t and a second kernel adds the partitions in a fixed order
 * (deterministic, no atomics); splits * B*H*N_Q*d floats per requested
 * gradient.  For small key grids with long query streams (few key-row
 * workgroups, each streaming many query tiles) the key gradients are
 * computed the same way by query partitions: splits * B*H*N_K*d floats per
 * requested gradient.  splits is the library's choice for these sizes; the
 * two halves run one after the other and share the workspace, whose size is
 * the larger of the two.  Where streamkl_bwd_fused_selected is 1 it is the
 * larger of that and streamkl_bwd_fused_workspace_size, so one workspace
 * serves streamkl_bwd, streamkl_bwd_dq_ws and streamkl_bwd_dk_ws alike.
 */
size_t streamkl_bwd_workspace_size(int B, int H, int N_Q, int N_K, int d,
                                   int causal, int dtype, int grad_mask);

/*
 * streamkl_bwd -- recompute backward pass ("Strategia di Ricalcolo", backward
 * pass section).  Regenerates P_t = exp(S_t - LSE_t) from the saved row
 * vectors and forms, for the upstream per-row gradient g = dkl (NULL = ones):
 *   dS2 = g (P2 - P1)                      (Configuration 1)
 *   dS1 = g P1 (S1 - S2 - (KL + LSE1 - LSE2))
 *       = g P1 (log P1 - log P2 - KL)      (Configuration 2; formed from
 *                                           logits and LSEs, never log P)
 *   dq_t = scale dS_t k_t,  dk_t = scale dS_t^T q_t.
 *   in : the forward inputs, kl/lse1/lse2 exactly as streamkl_fwd wrote them,
 *        dkl [B,H,N_Q] float32 or NULL, grad_mask (STREAMKL_GRAD_*).
 *   out: dq1, dk1 (required iff grad_mask has Q1K1), dq2, dk2 (iff Q2K2);
 *        pointers of unrequested gradients may be NULL and are not touched.
 *   workspace / workspace_bytes: at least streamkl_bwd_workspace_size(...)
 *        bytes, 16-byte aligned (may be NULL when that is 0), owned by the
 *        caller; its contents are dead once the call's work has completed.
 * With N_Q == 0 the key gradients are written as zeros.
 * Form: where streamkl_bwd_fused_selected(...) is 1 (bf16, short query
 * blocks, query-gradient buffer within L2) this is streamkl_bwd_fused;
 * otherwise the two-kernel form, streamkl_bwd_dk_ws then streamkl_bwd_dq_ws,
 * whose results are bitwise reproducible.
 */
streamkl_status streamkl_bwd(const void *q1, const void *k1, const void *q2,
                             const void *k2, const float *kl,
                             const float *lse1, const float *lse2,
                             const float *dkl, int B, int H, int N_Q, int N_K,
                             int d, float scale, int causal, int dtype,
                             int grad_mask, void *dq1, void *dk1, void *dq2,
                             void *dk2, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * streamkl_bwd_dq / streamkl_bwd_dk -- the two halves of streamkl_bwd, for
 * callers that schedule them separately (e.g. on two streams).  Same
 * arguments, meaning and errors as streamkl_bwd, restricted to the query
 * gradients (dq1, dq2) or to the key gradients (dk1, dk2).  Neither takes a
 * workspace: streamkl_bwd_dq never partitions the keys, nor streamkl_bwd_dk
 * the queries.  The page describes
 * this split as the fallback of its fused backward when atomic contention on
 * dQ is high ("Strategia di Ricalcolo", kernel fusion bullet).
 *
 * streamkl_bwd_dq_ws / streamkl_bwd_dk_ws -- the two halves with
 * streamkl_bwd's workspace: workspace / workspace_bytes as for streamkl_bwd
 * (at least streamkl_bwd_workspace_size(...) bytes for the same sizes and
 * grad_mask, 16-byte aligned, caller-owned, STREAMKL_ERR_WORKSPACE
 * otherwise).  Where the library partitions that half's streamed rows (the
 * keys of short query blocks, the queries of small key grids with long
 * query streams) the gradients are computed by partitions, partial sums in
 * the workspace, added in a fixed order; otherwise they are streamkl_bwd_dq
 * and streamkl_bwd_dk.  The two halves must not run at the same time on one
 * workspace.  Where the fused form is not selected, streamkl_bwd is
 * streamkl_bwd_dk_ws followed by streamkl_bwd_dq_ws on one stream, with
 * bitwise the same results; where it is, the two halves remain a
 * deterministic alternative to it.
 */
streamkl_status streamkl_bwd_dq(const void *q1, const void *k1, const void *q2,
                                const void *k2, const float *kl,
                                const float *lse1, const float *lse2,
                                const float *dkl, int B, int H, int N_Q,
                                int N_K, int d, float scale, int causal,
                                int dtype, int grad_mask, void *dq1, void *dq2,
                                void *stream);
streamkl_status streamkl_bwd_dq_ws(const void *q1, const void *k1,
                                   const void *q2, const void *k2,
                                   const float *kl, const float *lse1,
                                   const float *lse2, const float *dkl, int B,
                                   int H, int N_Q, int N_K, int d, float scale,
                                   int causal, int dtype, int grad_mask,
                                   void *dq1, void *dq2, void *workspace,
                                   size_t workspace_bytes, void *stream);
streamkl_status streamkl_bwd_dk(const void *q1, const void *k1, const void *q2,
                                const void *k2, const float *kl,
                                const float *lse1, const float *lse2,
                                const float *dkl, int B, int H, int N_Q,
                                int N_K, int d, float scale, int causal,
                                int dtype, int grad_mask, void *dk1, void *dk2,
                                void *stream);
streamkl_status streamkl_bwd_dk_ws(const void *q1, const void *k1,
                                   const void *q2, const void *k2,
                                   const float *kl, const float *lse1,
                                   const float *lse2, const float *dkl, int B,
                                   int H, int N_Q, int N_K, int d, float scale,
                                   int causal, int dtype, int grad_mask,
                                   void *dk1, void *dk2, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * streamkl_bwd_fused_workspace_size -- bytes of device workspace
 * streamkl_bwd_fused needs: one fp32 [B, H, N_Q, d] array per requested query
 * gradient (the sums its atomics add into).  0 for STREAMKL_F32 (not
 * supported by the fused form), for invalid sizes and for N_Q == 0.
 */
size_t streamkl_bwd_fused_workspace_size(int B, int H, int N_Q, int N_K,
                                         int d, int causal, int dtype,
                                         int grad_mask);

/*
 * streamkl_bwd_fused_selected -- 1 where streamkl_bwd runs the fused form:
 * the page's criterion (the query-gradient buffer, one fp32 [B, H, N_Q, d]
 * array per requested gradient, fits in the 32 MiB of L2 of the eight XCDs),
 * bf16 inputs, and short query blocks where it measured faster than the
 * two-kernel form: 1 <= N_Q <= 64 (one query tile per head); 0 otherwise.
 */
int streamkl_bwd_fused_selected(int B, int H, int N_Q, int N_K, int d,
                                int causal, int dtype, int grad_mask);

/*
 * streamkl_bwd_fused -- the single-pass recompute backward ("Strategia di
 * Ricalcolo", kernel-fusion bullet: each (query tile, key tile) pair is
 * visited once, key gradients are kept in registers and query gradients are
 * added with atomics into a buffer; the page's ablation bullet of
 * "Risultati Sperimentali" finds it faster for short query blocks).
 * Same arguments, meaning and results as streamkl_bwd, for bf16 inputs only:
 *   workspace / workspace_bytes: at least streamkl_bwd_fused_workspace_size
 *        bytes, 16-byte aligned, owned by the caller; cleared and written by
 *        the call, dead once its work has completed on `stream`.
 * Each pair's recompute is done once (12 d flops per admissible pair instead
 * of the two-kernel form's 16).  The fp32 additions of the query gradients
 * happen in a varying order, so dq1 / dq2 can differ in the last bits from
 * run to run; dk1 / dk2 are bitwise reproducible.
 * Errors as streamkl_bwd, plus STREAMKL_ERR_UNSUPPORTED for STREAMKL_F32 and
 * STREAMKL_ERR_WORKSPACE for a missing, misaligned or short workspace.
 */
streamkl_status streamkl_bwd_fused(const void *q1, const void *k1,
                                   const void *q2, const void *k2,
                                   const float *kl, const float *lse1,
                                   const float *lse2, const float *dkl, int B,
                                   int H, int N_Q, int N_K, int d, float scale,
                                   int causal, int dtype, int grad_mask,
                                   void *dq1, void *dk1, void *dq2, void *dk2,
                                   void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Static, human-readable name of a status code. */
const char *streamkl_status_str(int status);

/* Version of this ABI (bumped on any incompatible change). */
int streamkl_abi_version(void);

#ifdef STREAMKL_DEBUG
/*
 * streamkl_debug_take -- debug builds only (the library compiled with
 * -DSTREAMKL_DEBUG, libstreamkl_debug.so); not exported by release builds.
 * There every global-memory access of the kernels, and the LDS accesses of
 * their tile loops, are checked against the extent of the buffer they
 * belong to.  An access found out of range is not made (a global load or
 * copy reads zeros, an LDS access goes to the start of the workgroup's LDS,
 * a store or atomic is dropped), so a faulty index cannot fault the GPU; the
 * kernels keep the site of the first one.  This call waits for the device
 * (hipDeviceSynchronize), returns that site and clears it: 0 for none, else
 * (file << 16) | line, with file 1 streamkl_fwd.hip, 2 streamkl_bwd.h,
 * 3 streamkl_bwd_fused.hip of the library's sources; ~0 when the device
 * could not be read.  The record is per process, shared by every call.
 */
unsigned streamkl_debug_take(void);
#endif

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
