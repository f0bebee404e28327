// streamkl_bwd.h -- recompute backward kernel template (gfx950), shared by the
// dQ and dK translation units.
//
// StreamKL summary page (gist.science 2606.20005), "Strategia di Ricalcolo":
// only KL, LSE1 and LSE2 per row survive the forward pass; the backward pass
// regenerates P_t = exp(S_t - LSE_t) tile by tile from them and the original
// Q, K, and produces the gradients of the two configurations the page names
// (Configuration 1: P1 fixed, train P2; Configuration 2: P2 fixed, train P1).
// For an upstream per-row gradient g, the partial derivatives of
// sum_i g_i KL_i with respect to the scaled logits are
//   dS2 = g (P2 - P1),      dS1 = g P1 (S1 - S2 - delta),
//   delta = KL + LSE1 - LSE2 = sum_j P1 (S1 - S2),
// i.e. dS1 = g P1 (log P1 - log P2 - KL) with the log-ratio formed from
// logits and saved LSEs, never from log P (the page's numerical-stability
// point).  Then dQ_t = scale dS_t K_t and dK_t = scale dS_t^T Q_t.
//
// The page's kernel uses one fused pass with dQ atomics when the dQ buffer
// fits in L2 and two separate kernels when contention is high.  This file is
// the separate-kernel form: one template, two roles.
//   ROLE_DQ: a workgroup owns 256 query rows ("stationary"; 128 for fp32
//            with d = 128) and streams key tiles ("streamed") up to its
//            causal frontier; it accumulates dQ.
//   ROLE_DK: a workgroup owns 256 key rows (128 for fp32 with d = 128; 64
//            in the paired layout for small grids) and streams query tiles
//            from its causal frontier to N_Q; it accumulates dK.
// Both recompute S1, S2; neither needs atomics, and results are bitwise
// deterministic.  For short query blocks the query-gradient role can also run
// by key partitions, and the key-gradient role of small grids with long
// query streams by query partitions (SPLIT below): partial sums in a caller's
// workspace, added in a fixed order by part_reduce_kernel.
//
// Per 32-row block of a streamed tile, each wave:
//   1. S_t^T block (32 streamed x 32 stationary) = Y_t X_t^T with the
//      stationary fragments X_t in registers (B operand) and the streamed
//      rows Y_t read from LDS (A operand): each lane owns one stationary row
//      and 16 streamed rows of the block;
//   2. P_t = exp2(s_t * scale*log2e - LSE_t*log2e) and, with raw dot products
//      s_t and delta' = delta / scale,
//        e2 = P2 - P1           (dS2 = g e2)
//        e1 = P1 (s1 - s2 - delta')    (dS1 = g scale e1),
//      g multiplied in per element only where it varies along the block's
//      rows (ROLE_DK with an upstream gradient), otherwise at the end;
//   3. dX_t^T (d x 32 stationary) += Y_t^T e_t: the A operand Y_t^T is read
//      from the same row-major LDS tile with transposing reads
//      (ds_read_b64_tr_b16), in the row order of e_t's registers, so e_t feeds
//      the product as the B operand with no shuffles.
// Tiles arrive in LDS by direct global->LDS copies, double buffered.
#pragma once

#include "streamkl_device.h"
#include "streamkl_launch.h"

#include <climits>
#include <cmath>
#include <type_traits>

namespace streamkl {

enum { ROLE_DQ = 0, ROLE_DK = 1 };

// PAIR (key-gradient role, bf16, both gradients, small grids): the two waves
// of a pair own the same 32 stationary rows.  Per streamed tile each
// recomputes the scores of one of the two 32-row blocks and forms e1, e2
// there; they swap one of the two through LDS, and then wave 0 accumulates
// the teacher's gradient and wave 1 the student's over both blocks, each
// starting with the block it scored.  A wave then holds one d x 32
// accumulator instead of two and both stationary fragments fit in registers
// at two waves per SIMD, in workgroups of 64 keys (two per CU).
// Otherwise every wave owns its own 32 stationary rows and accumulates what
// is asked for; the teacher's stationary fragments live in an LDS tile
// wherever two waves per SIMD need the registers (workgroups of 8 waves, 256
// rows, one per CU).  For the key-gradient role this one-barrier-per-tile
// layout is 4-10% faster on large grids with long query streams; the paired
// one, with 4x the workgroups, wins on small grids (bwd_dk_paired below).
template <bool BF16, int D, bool PAIR>
struct BwdCfg {
  using G = RowGeom<BF16, D>;
  static_assert(!PAIR || BF16, "the paired layout is for bf16");
  static constexpr bool kX1Lds = !PAIR && (BF16 || D == 64);
  // Paired: four waves (two pairs, 64 stationary keys) and two workgroups
  // per CU -- barriers then wait for four waves, not eight.
  static constexpr int kWaves = PAIR ? 4 : kX1Lds ? 8 : 4;
  static constexpr int kWavesPerEU = (PAIR || kX1Lds) ? 2 : 1;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBS = 32 * (PAIR ? kWaves / 2 : kWaves);  // stationary rows per workgroup
  static constexpr int kBT = BF16 ? 64 : 32;              // streamed rows per LDS tile
  static constexpr int kSub = kBT / 32;                   // 32-row blocks per tile
  static_assert(!PAIR || kSub == 2, "a pair splits a tile's two blocks");
  static constexpr int kTileChunks = kBT * G::kChunks;    // 16-B chunks per tensor tile
  static constexpr int kLoads = kTileChunks / kThreads;   // copies per thread per tensor
  static constexpr int kXChunks = kX1Lds ? kBS * G::kChunks : 0;  // stationary teacher tile
  static constexpr int kXLoads = kXChunks / kThreads;
  static constexpr int kNCst = 4;                         // per-row constant arrays
  static constexpr int kOffY2 = kTileChunks;              // Y2 within a stage
  static constexpr int kStage = 2 * kTileChunks;          // one stage: (Y1, Y2) tiles
  static constexpr int kCstChunks = 2 * kNCst * kBT * int(sizeof(float)) / 16;  // both stages' constants
  static constexpr size_t kLdsBytes = size_t(kCstChunks + 2 * kStage + kXChunks + (PAIR ? kWaves * 128 : 0)) * 16;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kTileChunks % kThreads == 0, "tile must split evenly over the workgroup");
  static_assert(kXChunks % kThreads == 0, "stationary tile must split evenly over the workgroup");
};

struct BwdParams {
  const char *q1, *k1, *q2, *k2;
  const float *kl, *lse1, *lse2, *dkl;
  char *dq1, *dk1, *dq2, *dk2;
  int nq, nk, nsb;    // nsb: stationary blocks per head
  float scale, c;     // c = scale * log2(e)
  float inv_scale;
  // Partitions of the streamed rows (1 = none).  With nsplit > 1 the
  // query-gradient role's partition s streams key tiles [s*tps, (s+1)*tps);
  // the key-gradient role's splits the workgroup's own query range (from its
  // causal frontier to N_Q) into nsplit runs of equal length, so that every
  // key block's partitions are about equally long.  Each writes its fp32
  // partial gradient (already scaled) to part_t[s][bh * rows + i][d], rows
  // the role's stationary rows per head; a second kernel sums the
  // partitions in order and converts.
  int nsplit, tps;
  float *part1, *part2;
  // Causal, unsplit: the stationary blocks' ranks are taken over each XCD's
  // heads (lf 1, longest_first) or over the whole grid (lf 2, rank_major)
  // instead of head by head (0).
  int lf;
#ifdef STREAMKL_DEBUG
  // Bytes of a query tensor, a key tensor, a row vector and the partial sums
  // (both gradients', from part_lo).
  size_t xq, xk, xr, xp;
  const float *part_lo;
#endif
};

// Per-row constants of the recompute.
//  ROLE_DQ (the lane's own query, in registers): L_t = LSE_t log2(e) so that
//    P_t = exp2(s_t c - L_t); g (1 without an upstream gradient);
//    dp = delta / scale with delta = KL + LSE1 - LSE2.  Rows past N_Q get
//    L_t = inf, which makes every P they enter zero.
//  ROLE_DK (streamed queries, in LDS per tile): the initial accumulators of
//    the score products are -LSE1/scale and (KL - LSE2)/scale, so they yield
//    s1' = s1 - LSE1/scale and s2'' = s2 + (KL - LSE2)/scale; then
//    P1 = exp2(s1' c), P2 = exp2(s2'' c - KL c/scale) and
//    s1 - s2 - delta/scale = s1' - s2''.  The per-element constants left are
//    kc = -KL c/scale (and g itself when g varies).
struct RowCst {
  float l1, l2, g, dp;
};

__device__ __forceinline__ RowCst row_constants(const BwdParams &p, size_t i, bool valid) {
  RowCst r{INFINITY, INFINITY, 0.f, 0.f};
  if (valid) {
    const float lse1 = *SK_G(&p.lse1[i], 4, p.lse1, p.xr, 2), lse2 = *SK_G(&p.lse2[i], 4, p.lse2, p.xr, 2);
    const float kl = *SK_G(&p.kl[i], 4, p.kl, p.xr, 2);
    r.g = p.dkl ? *SK_G(&p.dkl[i], 4, p.dkl, p.xr, 2) : 1.f;
    r.l1 = lse1 * kLog2e;
    r.l2 = lse2 * kLog2e;
    r.dp = (kl + lse1 - lse2) * p.inv_scale;
  }
  return r;
}

// PO ("paired order"): the key-gradient role on a grid small enough for the
// paired layout.  With both gradients it selects that layout; with the
// student's gradient alone it takes the streamed blocks in the order the
// paired student wave does, so that both give the same bits.  The
// query-gradient role always runs one wave per 32 stationary rows.
template <bool BF16, int MASK, int ROLE, bool PO>
constexpr bool kPairOf = PO && BF16 && MASK == 3 && ROLE == ROLE_DK;

template <bool BF16, int D, int MASK, int ROLE, bool PO = false>
using BwdCfgOf = BwdCfg<BF16, D, kPairOf<BF16, MASK, ROLE, PO>>;

// Whether the key-gradient role takes the paired layout (bf16, both
// gradients).  The unpaired layout -- one 256-key workgroup per CU, which
// loads its 256 stationary keys before streaming -- needs at least two rounds
// of workgroups and query streams of 8192 rows to pay off.  Measured (dK
// kernel, causal, d = 128 unless stated; paired / unpaired time):
//   H x N = 8 x 2048: 0.51;  32 x 2048: 0.86;  16 x 4096: 0.75;
//   8 x 8192: 0.77;  32 x 4096: 0.84;  16 x 8192: 1.04;  64 x 8192: 1.04;
//   4 x 32768: 1.08;  2 x 65536: 1.10;  32 x 8192 (d = 64): 1.09.
inline bool bwd_dk_paired(int bh, int nq, int nk, bool bf16) {
  if (!bf16) return false;
  const long long unpaired = (long long)bh * ((nk + 255) / 256);
  return unpaired < 2 * 256 || nq < 8192;
}

// SPLIT: the workgroup folds one partition of its streamed rows and stores
// fp32 partial gradients instead of the gradients themselves.
template <bool BF16, int D, bool CAUSAL, int ROLE, int MASK, bool GSIGN, bool SPLIT, bool PO>
__global__ __attribute__((amdgpu_flat_work_group_size(BwdCfgOf<BF16, D, MASK, ROLE, PO>::kThreads,
                                                      BwdCfgOf<BF16, D, MASK, ROLE, PO>::kThreads),
                          amdgpu_waves_per_eu(BwdCfgOf<BF16, D, MASK, ROLE, PO>::kWavesPerEU,
                                              BwdCfgOf<BF16, D, MASK, ROLE, PO>::kWavesPerEU)))
void bwd_kernel(BwdParams p) {
  using C = BwdCfgOf<BF16, D, MASK, ROLE, PO>;
  using G = typename C::G;
  constexpr bool kPair = kPairOf<BF16, MASK, ROLE, PO>;
  constexpr bool kG1 = (MASK & 1) != 0;
  constexpr bool kG2 = (MASK & 2) != 0;
  constexpr int kMB = D / 32;  // 32-row blocks of d in the gradient accumulators
  // LDS: the row constants, the stages and the stationary tile at fixed
  // offsets of one dynamic array, the pairs' exchange slots in a static one.
  // From the constant offsets the compiler can tell that reading one stage
  // (or the constants, the stationary tile, the slots) need not wait for the
  // copies in flight into the other stage.  The constants come first: every
  // read of them is then one lane offset plus an immediate below 64 KB.
  extern __shared__ u32x4 lds[];
  float (*cstage)[C::kNCst * C::kBT] = reinterpret_cast<float (*)[C::kNCst * C::kBT]>(lds);
  u32x4 *ystage0 = lds + C::kCstChunks, *ystage1 = ystage0 + C::kStage;
  u32x4 *xtile = ystage0 + 2 * C::kStage;
  __shared__ u32x4 xch[kPair ? C::kWaves * 128 : 1];          // pairs' exchange slots

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  // The wave's 32 stationary rows within the workgroup and, in a pair, the
  // streamed block it scores and the gradient it accumulates (0: teacher).
  const int wrow = kPair ? wave >> 1 : wave;
  const int half = kPair ? wave & 1 : 0;

  // With key partitions, the stationary blocks of one (head, partition) are
  // consecutive, so they share the partition's tiles in one L2.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_bh = SPLIT ? p.nsb * p.nsplit : p.nsb;
  int bh = bid / per_bh;
  const int rem = bid - bh * per_bh;
  const int split = SPLIT ? rem / p.nsb : 0;
  int sbr = rem - split * p.nsb;
  // Longest rows first: for causal problems the last query blocks (ROLE_DQ)
  // and the first key blocks (ROLE_DK) see the most partners; with p.lf the
  // ranks are taken over the XCD's heads (longest_first) or over the whole
  // grid (rank_major).
  if (CAUSAL && !SPLIT && p.lf) {
    const BlockPos bp = p.lf == 1 ? longest_first(bid, gridDim.x, p.nsb)
                                  : rank_major(blockIdx.x, gridDim.x / p.nsb);
    bh = bp.bh;
    sbr = bp.rank;
  }
  const int sblk = (CAUSAL && ROLE == ROLE_DQ) ? p.nsb - 1 - sbr : sbr;

  const int ns = ROLE == ROLE_DQ ? p.nq : p.nk;  // stationary rows per head
  const int nt = ROLE == ROLE_DQ ? p.nk : p.nq;  // streamed rows per head
  const int off = p.nk - p.nq;
  const char *X1 = ROLE == ROLE_DQ ? p.q1 : p.k1;
  const char *X2 = ROLE == ROLE_DQ ? p.q2 : p.k2;
  const char *Y1 = (ROLE == ROLE_DQ ? p.k1 : p.q1) + size_t(bh) * nt * G::kRowBytes;
  const char *Y2 = (ROLE == ROLE_DQ ? p.k2 : p.q2) + size_t(bh) * nt * G::kRowBytes;
  const size_t xoff = size_t(bh) * ns * G::kRowBytes;

  const int s0 = sblk * C::kBS;
  const int w0 = s0 + wrow * 32;
  const int srow = w0 + col;
#ifdef STREAMKL_DEBUG
  // Extents of the stationary and streamed tensors, and of the dynamic LDS.
  const size_t xS = ROLE == ROLE_DQ ? p.xq : p.xk, xT = ROLE == ROLE_DQ ? p.xk : p.xq;
  const char *T1 = ROLE == ROLE_DQ ? p.k1 : p.q1, *T2 = ROLE == ROLE_DQ ? p.k2 : p.q2;
  constexpr size_t kDyn = size_t(2 * C::kStage + C::kXChunks) * 16 + 2 * C::kNCst * C::kBT * 4;
#endif

  // Stationary fragments (B operand of the score products): the student's in
  // registers; the teacher's in registers or, with kX1Lds, in the LDS tile
  // filled below.  Rows past the end are zero (registers) or repeat the last
  // row (LDS); neither is ever written out.
  constexpr int kX1Regs = C::kX1Lds ? 1 : G::kLaneChunks;
  u32x4 xf1[kX1Regs], xf2[G::kLaneChunks];
  if (srow < ns) {
    const u32x4 *r1 = reinterpret_cast<const u32x4 *>(X1 + xoff + size_t(srow) * G::kRowBytes);
    const u32x4 *r2 = reinterpret_cast<const u32x4 *>(X2 + xoff + size_t(srow) * G::kRowBytes);
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) {
      if (!C::kX1Lds) xf1[c] = *SK_G((&r1[frag_chunk<BF16, D>(h, c)]), 16, X1, xS, 2);
      xf2[c] = *SK_G((&r2[frag_chunk<BF16, D>(h, c)]), 16, X2, xS, 2);
    }
  } else {
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) {
      if (!C::kX1Lds) xf1[c] = zero4();
      xf2[c] = zero4();
    }
  }
  if constexpr (C::kX1Lds) {
    // the workgroup's stationary teacher rows -> LDS (swizzled like the tiles)
#pragma unroll
    for (int i = 0; i < C::kXLoads; ++i) {
      const int pos = i * C::kThreads + tid;
      const int row = pos / G::kChunks;
      const int ch = swz<G::kChunks>(row, pos % G::kChunks);
      const int r = min(s0 + row, ns - 1);
      dma16(SK_G(X1 + xoff + size_t(r) * G::kRowBytes + ch * 16, 16, X1, xS, 2),
            SK_L(xtile + i * C::kThreads + wave * 64, 1024, lds, kDyn, 2));
    }
  }

  // ROLE_DQ: the lane's query is stationary; its constants live in registers.
  RowCst rc{INFINITY, INFINITY, 0.f, 0.f};
  if (ROLE == ROLE_DQ) rc = row_constants(p, size_t(bh) * p.nq + srow, srow < p.nq);

  // Streamed range and per-element admissibility.
  //   ROLE_DQ (streamed keys tau, stationary query sigma): tau <= sigma + off, tau < N_K.
  //   ROLE_DK (streamed queries tau, stationary key sigma): tau >= sigma - off, tau < N_Q.
  int t_begin = 0, t_end = nt;
  if (CAUSAL) {
    if (ROLE == ROLE_DQ) t_end = min(p.nk, min(s0 + C::kBS, p.nq) + off);
    else t_begin = max(0, s0 - off);
  }
  int tile0 = t_begin / C::kBT;
  int tile1 = (t_end + C::kBT - 1) / C::kBT;
  if (SPLIT) {  // this partition's share of the tiles
    if (ROLE == ROLE_DQ) {
      tile0 = max(tile0, split * p.tps);
      tile1 = min(tile1, (split + 1) * p.tps);
    } else if (tile1 > tile0) {
      const int len = (tile1 - tile0 + p.nsplit - 1) / p.nsplit;
      tile0 += split * len;
      tile1 = min(tile1, tile0 + len);
    }
  }
  // ROLE_DQ: last admissible key; ROLE_DK: first admissible query.
  const int lim = ROLE == ROLE_DQ ? (CAUSAL ? min(srow + off, p.nk - 1) : p.nk - 1)
                                  : (CAUSAL ? max(srow - off, 0) : 0);

  // ------------------------------------------------------------ staging
  // Streamed tile `tile` -> LDS buffer `stage` by direct global->LDS copies.
  // Lane L of wave w fills chunk position i*threads + 64w + L; the global side
  // picks the (row, logical chunk) stored there (the swizzle is an XOR, its
  // own inverse).  Rows past the end repeat the last row; they are masked.
  // Full tiles take 32-bit offsets from the head's base (where a head's rows
  // span fewer than 2^32 bytes): one per copy, a constant apart.  The last
  // tile, and heads of 4 GiB or more, use 64-bit offsets and clamp each row.
  // The key-gradient role issues its 32-bit-offset copies unseen by the
  // compiler (dma16_unseen): its transposing reads carry no alias
  // information, so a visible copy would make the first of them wait for the
  // copy in flight, and every LDS wait meanwhile would be lgkmcnt(0).  The
  // query-gradient role measured no faster that way and keeps the builtin.
  constexpr bool kUnseen = ROLE == ROLE_DK;
  const bool off32 = size_t(nt) * G::kRowBytes <= size_t(0xFFFFFFFFu);
  auto issue = [&](int tile, int stage) {
    u32x4 *wbase = (stage ? ystage1 : ystage0) + wave * 64;
    if (off32 && (tile + 1) * C::kBT <= nt) {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        const int pos = i * C::kThreads + tid;
        const int row = pos / G::kChunks;
        const int ch = swz<G::kChunks>(row, pos % G::kChunks);
        const uint32_t o = uint32_t(tile * C::kBT + row) * G::kRowBytes + uint32_t(ch * 16);
#ifdef STREAMKL_DEBUG
        // Checked copies are issued through the builtin; the explicit waits
        // of the unseen form stay in place.
        dma16(SK_G(Y1 + o, 16, T1, xT, 2), SK_L(wbase + i * C::kThreads, 1024, lds, kDyn, 2));
        dma16(SK_G(Y2 + o, 16, T2, xT, 2), SK_L(wbase + i * C::kThreads + C::kOffY2, 1024, lds, kDyn, 2));
#else
        if constexpr (kUnseen) {
          dma16_unseen(Y1, o, wbase + i * C::kThreads);
          dma16_unseen(Y2, o, wbase + i * C::kThreads + C::kOffY2);
        } else {
          dma16(Y1 + o, wbase + i * C::kThreads);
          dma16(Y2 + o, wbase + i * C::kThreads + C::kOffY2);
        }
#endif
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        const int pos = i * C::kThreads + tid;
        const int row = pos / G::kChunks;
        const int ch = swz<G::kChunks>(row, pos % G::kChunks);
        const int r = min(tile * C::kBT + row, nt - 1);
        const size_t o = size_t(r) * G::kRowBytes + ch * 16;
        dma16(SK_G(Y1 + o, 16, T1, xT, 2), SK_L(wbase + i * C::kThreads, 1024, lds, kDyn, 2));
        dma16(SK_G(Y2 + o, 16, T2, xT, 2), SK_L(wbase + i * C::kThreads + C::kOffY2, 1024, lds, kDyn, 2));
      }
    }
  };
  // ROLE_DK: the next tile's per-row inputs, loaded while the current tile is
  // processed and turned into constants only at the end of the step, so the
  // wait for these loads does not also wait for the tile copies behind them.
  float n_lse1 = 0.f, n_lse2 = 0.f, n_kl = 0.f, n_g = 0.f;
  bool n_ok = false;
  auto cload = [&](int tile) {
    if (ROLE == ROLE_DK && tid < C::kBT) {
      const int row = tile * C::kBT + tid;
      n_ok = row < p.nq;
      if (n_ok) {
        const size_t i = size_t(bh) * p.nq + row;
        n_lse1 = *SK_G(&p.lse1[i], 4, p.lse1, p.xr, 2);
        n_lse2 = *SK_G(&p.lse2[i], 4, p.lse2, p.xr, 2);
        n_kl = *SK_G(&p.kl[i], 4, p.kl, p.xr, 2);
        n_g = p.dkl ? *SK_G(&p.dkl[i], 4, p.dkl, p.xr, 2) : 1.f;
      }
    }
  };
  auto cstore = [&](int stage) {
    if (ROLE == ROLE_DK && tid < C::kBT) {
      // Rows past N_Q: -1e30 (not -inf) keeps s1' - s2'' finite (0) and P = 0.
      float *cst = SK_L(cstage[stage], C::kNCst * C::kBT * 4, lds, kDyn, 2);
      cst[tid] = n_ok ? -n_lse1 * p.inv_scale : -1e30f;
      cst[C::kBT + tid] = n_ok ? (n_kl - n_lse2) * p.inv_scale : -1e30f;
      cst[2 * C::kBT + tid] = n_ok ? n_g : 0.f;
      cst[3 * C::kBT + tid] = n_ok ? -n_kl * p.inv_scale * p.c : 0.f;
    }
  };

  // Byte offsets of the transposing reads of the gradient products (bf16)
  // at block 0, k-step 0, per 32-column block mb of d and row half t (see
  // grad_bf16 below).  The swizzle depends on row bits 0-3 only, so the other
  // blocks and k-steps (multiples of 16 rows) add a constant.
  int trofs[kMB][2];
  {
    const int s16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int d0 = mb * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
        const int row = 8 * t + 4 * h + (s16 >> 2);
        trofs[mb][t] = (row * G::kChunks + swz<G::kChunks>(row, d0 >> 3)) * 16 + (d0 & 7) * 2;
      }
  }

  f32x16 acc1[kMB], acc2[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    acc1[mb] = f32x16{};
    acc2[mb] = f32x16{};
  }

  const float c = p.c;
  const int ntiles = max(tile1 - tile0, 0);
  if (ntiles > 0) {
    cload(tile0);
    issue(tile0, 0);
    cstore(0);
  }
  if constexpr (kUnseen) vmcnt0_wait();  // copies the compiler's own waits do not cover
  __syncthreads();

  // e1/e2 of one 32-row block in the form the gradient product consumes:
  // packed bf16 B operands for the two 16-row k-steps, or fp32 values.
  struct EBlock {
    u32x4 pk1[2], pk2[2];
    float e1[16], e2[16];
  };

  // One streamed tile.  `stage_c` is the LDS buffer as a compile-time
  // constant, so every LDS address below is a loop-invariant lane offset plus
  // an immediate; the loop is unrolled by two to alternate the buffers.
  auto tile_step = [&](int it, auto stage_c, auto half_c) {
    constexpr int stage = decltype(stage_c)::value;
    constexpr int hc = decltype(half_c)::value;  // the wave's half of a pair, as a constant
    const int tile = tile0 + it;
    // Buffer stage^1 was last read in iteration it-1, which ended in a barrier.
    if (it + 1 < ntiles) {
      cload(tile + 1);
      issue(tile + 1, stage ^ 1);
    }
    const u32x4 *ybase = stage ? ystage1 : ystage0;
    const float *cst = SK_L(cstage[stage], C::kNCst * C::kBT * 4, lds, kDyn, 2);

    // Whether block sb holds an inadmissible (streamed, stationary) pair for
    // any lane of this wave: a causal frontier or the end of the streamed rows
    // passes through it (wave-uniform).
    auto straddles = [&](int sb) {
      const int tb = tile * C::kBT + sb * 32;
      if (ROLE == ROLE_DQ) return tb + 31 > (CAUSAL ? min(w0 + off, p.nk - 1) : p.nk - 1);
      return tb + 31 > p.nq - 1 || (CAUSAL && tb < max(w0 + 31 - off, 0));
    };

    // 1. recompute the two score blocks of block sb.  Inadmissible pairs start
    //    from -1e30 instead of their row constant: their P is then exactly 0
    //    and s1 - s2 is 0 (both products are absorbed), so e1 = e2 = 0 with no
    //    mask in the per-element work.  Only blocks that straddle pay for it.
    auto scores = [&](int sb, f32x16 &s1, f32x16 &s2, bool masked) {
      if (ROLE == ROLE_DK) {
        // initial accumulators of the block's rows, in C layout
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = sb * 32 + g4 * 8 + 4 * h;
          const f32x4 v1 = *reinterpret_cast<const f32x4 *>(cst + r0);
          const f32x4 v2 = *reinterpret_cast<const f32x4 *>(cst + C::kBT + r0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s1[4 * g4 + q] = v1[q];
            s2[4 * g4 + q] = v2[q];
          }
        }
      } else {
        s1 = f32x16{};
        s2 = f32x16{};
      }
      if (masked) {
        // Element r sits at streamed row rel + c_row(r, 0).
        const int rel = tile * C::kBT + sb * 32 + 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = rel + c_row(r, 0);
          const bool ok = ROLE == ROLE_DQ ? t <= lim : (t >= lim && t < p.nq);
          s1[r] = ok ? s1[r] : -1e30f;
          s2[r] = ok ? s2[r] : -1e30f;
        }
      }
      const int arow = sb * 32 + col;
      const int xrow = wrow * 32 + col;  // the lane's stationary row in the LDS tile
      if constexpr (kPair) {
        // The fragments are read one chunk ahead of their products, into a
        // second pair of registers, so the products of one chunk run while
        // the next chunk's reads are in flight.
        constexpr int kAhead = 1;
        u32x4 f1[kAhead + 1], f2[kAhead + 1];
        auto frag = [&](int cc) {
          const int pos = arow * G::kChunks + swz<G::kChunks>(arow, frag_chunk<BF16, D>(h, cc));
          f1[cc % (kAhead + 1)] = *SK_L(&ybase[pos], 16, lds, kDyn, 2);
          f2[cc % (kAhead + 1)] = *SK_L(&ybase[C::kOffY2 + pos], 16, lds, kDyn, 2);
        };
#pragma unroll
        for (int cc = 0; cc < kAhead; ++cc) frag(cc);
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          if (cc + kAhead < G::kLaneChunks) frag(cc + kAhead);
          mfma_chunk<BF16>(f1[cc % (kAhead + 1)], xf1[cc], s1);
          mfma_chunk<BF16>(f2[cc % (kAhead + 1)], xf2[cc], s2);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);  // the first chunks' reads
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          if (cc + kAhead < G::kLaneChunks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);          // chunk cc's products
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // Without pairing, the MFMA bursts run at raised priority so that the
        // other wave on the SIMD keeps the vector unit busy meanwhile (paired
        // waves gain nothing from it).
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          const int fc = frag_chunk<BF16, D>(h, cc);
          const int pos = arow * G::kChunks + swz<G::kChunks>(arow, fc);
          if constexpr (C::kX1Lds) {
            const u32x4 x1 = *SK_L((&xtile[xrow * G::kChunks + swz<G::kChunks>(xrow, fc)]), 16, lds, kDyn, 2);
            mfma_chunk<BF16>(*SK_L(&ybase[pos], 16, lds, kDyn, 2), x1, s1);
          } else {
            mfma_chunk<BF16>(*SK_L(&ybase[pos], 16, lds, kDyn, 2), xf1[cc], s1);
          }
          mfma_chunk<BF16>(*SK_L(&ybase[C::kOffY2 + pos], 16, lds, kDyn, 2), xf2[cc], s2);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    };

    // 2. regenerate P and form e1, e2 (fp32).
    auto form = [&](int sb, const f32x16 &s1, const f32x16 &s2, EBlock &E) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 Gv, KCv;
        if (ROLE == ROLE_DK) {
          const int r0 = sb * 32 + g4 * 8 + 4 * h;
          if (GSIGN) Gv = *reinterpret_cast<const f32x4 *>(cst + 2 * C::kBT + r0);
          KCv = *reinterpret_cast<const f32x4 *>(cst + 3 * C::kBT + r0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = g4 * 4 + q;
          if (ROLE == ROLE_DK) {  // s1' and s2'' carry their row constants
            const float p1 = fast_exp2(s1[r] * c);
            const float p2 = kG2 ? fast_exp2(fmaf(s2[r], c, KCv[q])) : 0.f;
            if (GSIGN) {
              const float gp1 = p1 * Gv[q];
              E.e2[r] = fmaf(p2, Gv[q], -gp1);
              E.e1[r] = gp1 * (s1[r] - s2[r]);
            } else {
              E.e2[r] = p2 - p1;
              E.e1[r] = p1 * (s1[r] - s2[r]);
            }
          } else {
            // ROLE_DQ: constants of the lane's own row; g is applied at write-out.
            const float p1 = fast_exp2(fmaf(s1[r], c, -rc.l1));
            const float p2 = kG2 ? fast_exp2(fmaf(s2[r], c, -rc.l2)) : 0.f;
            E.e2[r] = p2 - p1;
            E.e1[r] = p1 * ((s1[r] - s2[r]) - rc.dp);
          }
        }
      }
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            E.pk1[ks][w] = pack_bf16(E.e1[8 * ks + 2 * w], E.e1[8 * ks + 2 * w + 1]);
            E.pk2[ks][w] = pack_bf16(E.e2[8 * ks + 2 * w], E.e2[8 * ks + 2 * w + 1]);
          }
      }
    };

    // 3. gradient products of block sb: dX_t^T += Y_t^T e_t.
    //    bf16: Y_t^T comes from transposing reads of the tile; lane (s, grp)
    //    (s = lane % 16, grp = lane / 16) supplies row sb*32 + 16ks + 8t +
    //    4h + s/4, columns mb*32 + 16(grp&1) + 4(s&3) .. +3.
    auto grad_bf16 = [&](int sb, const char *yb, const u32x4 (&pk)[2], f32x16 (&acc)[kMB]) {
      const int s16 = lane & 15, grp = lane >> 4;
      if (!kPair) __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          const int d0 = mb * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
          u32x4 a;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            // The paired kernel schedules better with the offset formed per
            // read; the others keep fewer address registers with the hoisted
            // offsets (measured).
            const int row = sb * 32 + 16 * ks + 8 * t + 4 * h + (s16 >> 2);
            const int byte = kPair ? (row * G::kChunks + swz<G::kChunks>(row, d0 >> 3)) * 16 + (d0 & 7) * 2
                                   : trofs[mb][t] + (sb * 32 + 16 * ks) * G::kRowBytes;
            const u32x2 v = read_tr(SK_L(yb + byte, 8, lds, kDyn, 2));
            a[2 * t] = v[0];
            a[2 * t + 1] = v[1];
          }
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, pk[ks]), acc[mb], 0, 0, 0);
        }
      if (!kPair) __builtin_amdgcn_s_setprio(0);
    };
    auto grad = [&](int sb, const EBlock &E) {
      if constexpr (BF16) {
        if (kG1) grad_bf16(sb, reinterpret_cast<const char *>(ybase), E.pk1, acc1);
        if (kG2) grad_bf16(sb, reinterpret_cast<const char *>(ybase + C::kOffY2), E.pk2, acc2);
      } else {
        const float *yf1 = reinterpret_cast<const float *>(ybase);
        const float *yf2 = reinterpret_cast<const float *>(ybase + C::kOffY2);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            const int d = mb * 32 + col;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int row = sb * 32 + 16 * ks + c_row(j, h);
              const int idx = (row * G::kChunks + swz<G::kChunks>(row, d >> 2)) * 4 + (d & 3);
              if (kG1)
                acc1[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(*SK_L(&yf1[idx], 4, lds, kDyn, 2), E.e1[8 * ks + j],
                                                                acc1[mb], 0, 0, 0);
              if (kG2)
                acc2[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(*SK_L(&yf2[idx], 4, lds, kDyn, 2), E.e2[8 * ks + j],
                                                                acc2[mb], 0, 0, 0);
            }
          }
      }
    };

    // Blocks wholly outside the admissible region contribute exact zeros.
    if constexpr (kPair) {
      f32x16 s1, s2;
      EBlock E;
      scores(hc, s1, s2, straddles(hc));
      form(hc, s1, s2, E);
      // Keep the operand of the gradient this wave accumulates; hand the
      // other to the partner, which scored the other block.
      u32x4 mine[2], theirs[2];
      u32x4 *slot = SK_L(xch + wave * 128 + lane, 64 * 16 + 16, xch, sizeof(xch), 2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        mine[ks] = hc ? E.pk2[ks] : E.pk1[ks];
        slot[64 * ks] = hc ? E.pk1[ks] : E.pk2[ks];
      }
      // Barrier that waits for this wave's LDS stores only (lgkmcnt), not
      // for the tile copies in flight; the empty asm statements keep the
      // compiler from moving memory accesses across it.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const u32x4 *peer = SK_L(xch + (wave ^ 1) * 128 + lane, 64 * 16 + 16, xch, sizeof(xch), 2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) theirs[ks] = peer[64 * ks];
      // Each wave adds its own block first, so its first products need no
      // data from the partner.  The student's gradient thus takes the blocks
      // in the order 1, 0, as the unpaired kernel does for it.
      const char *yb = reinterpret_cast<const char *>(ybase + hc * C::kOffY2);
      grad_bf16(hc, yb, mine, acc1);
      grad_bf16(1 - hc, yb, theirs, acc1);
    } else {
      // The key-gradient role with the student's gradient alone, on a grid
      // where both gradients take the paired layout, takes the blocks in the
      // order the paired kernel's student wave does (its own block, 1,
      // first), so both give the same bits.
      constexpr bool kRev = PO && BF16 && ROLE == ROLE_DK && MASK == 2;
#pragma unroll
      for (int i = 0; i < C::kSub; ++i) {
        const int sb = kRev ? C::kSub - 1 - i : i;
        f32x16 s1, s2;
        EBlock E;
        scores(sb, s1, s2, straddles(sb));
        form(sb, s1, s2, E);
        grad(sb, E);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (it + 1 < ntiles) cstore(stage ^ 1);
    if constexpr (kUnseen) vmcnt0_wait();  // the copies into stage^1
    __syncthreads();  // also waits for the copies the compiler sees
  };

  auto run = [&](auto half_c) {
    for (int it = 0; it < ntiles; it += 2) {
      tile_step(it, std::integral_constant<int, 0>{}, half_c);
      if (it + 1 < ntiles) tile_step(it + 1, std::integral_constant<int, 1>{}, half_c);
    }
  };
  // A pair's two waves run their own copy of the loop, in which the half is a
  // constant: which operand a wave keeps, hands over and adds first is then
  // fixed.  (half is wave-uniform.)
  if constexpr (kPair) {
    if (half) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }

  // ---------------------------------------------------------------- write-out
  // dS2 = g e2 and dS1 = g scale e1; the gradients carry one more scale.
  if (srow < ns) {
    const float gq = ROLE == ROLE_DQ ? rc.g : 1.f;
    const float f1 = p.scale * p.scale * gq, f2 = p.scale * gq;
    const size_t ro = (size_t(bh) * ns + srow) * G::kRowBytes;
    char *O1 = (ROLE == ROLE_DQ ? p.dq1 : p.dk1) + ro;
    char *O2 = (ROLE == ROLE_DQ ? p.dq2 : p.dk2) + ro;
#ifdef STREAMKL_DEBUG
    const char *O1b = ROLE == ROLE_DQ ? p.dq1 : p.dk1, *O2b = ROLE == ROLE_DQ ? p.dq2 : p.dk2;
#endif
    auto store = [&](char *O, float f, const f32x16 (&A)[kMB] SK_DBG_ARGS(const char *Obase)) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = mb * 32 + g4 * 8 + 4 * h;
          const float v0 = A[mb][4 * g4] * f, v1 = A[mb][4 * g4 + 1] * f;
          const float v2 = A[mb][4 * g4 + 2] * f, v3 = A[mb][4 * g4 + 3] * f;
          if constexpr (BF16) {
            if (SK_OK(O + d0 * 2, 8, Obase, xS, 2))
              *reinterpret_cast<u32x2 *>(O + d0 * 2) = u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
          } else {
            if (SK_OK(O + d0 * 4, 16, Obase, xS, 2)) *reinterpret_cast<f32x4 *>(O + d0 * 4) = f32x4{v0, v1, v2, v3};
          }
        }
    };
    // A key partition's share: scaled fp32 partial sums, d values per row.
    auto store_part = [&](float *P, float f, const f32x16 (&A)[kMB]) {
      float *row = P + (size_t(split) * (size_t(gridDim.x / per_bh) * ns) + size_t(bh) * ns + srow) * D;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = mb * 32 + g4 * 8 + 4 * h;
          if (SK_OK(row + d0, 16, p.part_lo, p.xp, 2))
            *reinterpret_cast<f32x4 *>(row + d0) =
                f32x4{A[mb][4 * g4] * f, A[mb][4 * g4 + 1] * f, A[mb][4 * g4 + 2] * f, A[mb][4 * g4 + 3] * f};
        }
    };
    if constexpr (kPair) {
      if (SPLIT) store_part(half ? p.part2 : p.part1, half ? f2 : f1, acc1);
      else store(half ? O2 : O1, half ? f2 : f1, acc1 SK_DBG_ARGS(half ? O2b : O1b));
    } else if (SPLIT) {
      if (kG1) store_part(p.part1, f1, acc1);
      if (kG2) store_part(p.part2, f2, acc2);
    } else {
      if (kG1) store(O1, f1, acc1 SK_DBG_ARGS(O1b));
      if (kG2) store(O2, f2, acc2 SK_DBG_ARGS(O2b));
    }
  }
}

// Sum of the partitions' partial gradients of one role (ROLE: the query
// gradients' key partitions or the key gradients' query partitions), in
// partition order (deterministic), converted to the gradient's element type.
// One thread per four consecutive values of one row; blockIdx.y picks the
// gradient, so both requested gradients take one launch.
template <bool BF16, int ROLE>
__global__ __launch_bounds__(256) void part_reduce_kernel(const float *__restrict__ part0, char *out0,
                                                        const float *__restrict__ part1, char *out1, int nsplit,
                                                        size_t n4 SK_DBG_ARGS(const float *plo, size_t xp, size_t xo)) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  const float *part = blockIdx.y ? part1 : part0;
  char *out = blockIdx.y ? out1 : out0;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(part) + i;
  f32x4 acc = *SK_G(src, 16, plo, xp, 2);
  for (int s = 1; s < nsplit; ++s) {
    const f32x4 v = *SK_G(&src[size_t(s) * n4], 16, plo, xp, 2);
    acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
  }
  if constexpr (BF16) {
    if (SK_OK(reinterpret_cast<u32x2 *>(out) + i, 8, out, xo, 2))
      reinterpret_cast<u32x2 *>(out)[i] = u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  } else {
    if (SK_OK(reinterpret_cast<f32x4 *>(out) + i, 16, out, xo, 2)) reinterpret_cast<f32x4 *>(out)[i] = acc;
  }
}

template <bool BF16, int D, bool CAUSAL, int ROLE, int MASK, bool GSIGN, bool PO>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  constexpr bool kCanSplit = true;
  using C = BwdCfgOf<BF16, D, MASK, ROLE, PO>;
  BwdParams p;
  p.q1 = static_cast<const char *>(a.q1);
  p.k1 = static_cast<const char *>(a.k1);
  p.q2 = static_cast<const char *>(a.q2);
  p.k2 = static_cast<const char *>(a.k2);
  p.kl = a.kl;
  p.lse1 = a.lse1;
  p.lse2 = a.lse2;
  p.dkl = a.dkl;
  p.dq1 = static_cast<char *>(a.dq1);
  p.dk1 = static_cast<char *>(a.dk1);
  p.dq2 = static_cast<char *>(a.dq2);
  p.dk2 = static_cast<char *>(a.dk2);
  p.nq = a.nq;
  p.nk = a.nk;
  const int ns = ROLE == ROLE_DQ ? a.nq : a.nk;
  p.nsb = (ns + C::kBS - 1) / C::kBS;
  p.scale = a.scale;
  p.c = float(double(a.scale) * 1.4426950408889634);
  p.inv_scale = float(1.0 / double(a.scale));
  const int splits = ROLE == ROLE_DQ ? a.dq_splits : a.dk_splits;
  const bool split = kCanSplit && splits > 1 && a.part != nullptr;
  p.nsplit = split ? splits : 1;
  p.tps = (((a.nk + C::kBT - 1) / C::kBT) + p.nsplit - 1) / p.nsplit;  // the query-gradient role's
  const size_t part_elems = size_t(a.bh) * ns * D * p.nsplit;  // per requested gradient
  p.part1 = split ? a.part : nullptr;
  p.part2 = split ? a.part + ((MASK & 1) ? part_elems : 0) : nullptr;
#ifdef STREAMKL_DEBUG
  p.xq = size_t(a.bh) * a.nq * C::G::kRowBytes;
  p.xk = size_t(a.bh) * a.nk * C::G::kRowBytes;
  p.xr = size_t(a.bh) * a.nq * sizeof(float);
  p.part_lo = a.part;
  p.xp = split ? part_elems * (((MASK & 1) ? 1 : 0) + ((MASK & 2) ? 1 : 0)) * sizeof(float) : 0;
#endif
  // Resident workgroups per XCD: 32 CUs x (4 SIMDs x waves per SIMD / waves).
  constexpr long long kResidentPerXcd = 32LL * (4 * C::kWavesPerEU / C::kWaves);
  const long long nwg_all = (long long)p.nsb * a.bh;
  p.lf = (!CAUSAL || split) ? 0
         : longest_first_pays(nwg_all, p.nsb, kResidentPerXcd) ? 1
         : rank_major_pays(nwg_all, p.nsb, kResidentPerXcd)    ? 2
                                                                : 0;
  const long long blocks = (long long)p.nsb * a.bh * p.nsplit;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const void *fn = split ? reinterpret_cast<const void *>(&bwd_kernel<BF16, D, CAUSAL, ROLE, MASK, GSIGN, kCanSplit, PO>)
                         : reinterpret_cast<const void *>(&bwd_kernel<BF16, D, CAUSAL, ROLE, MASK, GSIGN, false, PO>);
  void *args[] = {&p};
  const size_t dyn = size_t(2 * C::kStage + C::kXChunks) * 16 + 2 * C::kNCst * C::kBT * 4;
  if (dyn > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn));
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(C::kThreads), args, dyn, stream);
  if (e != hipSuccess || !split) return e;
  const size_t n4 = size_t(a.bh) * ns * D / 4;
  const size_t rblocks = (n4 + 255) / 256;
  if (rblocks > size_t(INT_MAX)) return hipErrorInvalidConfiguration;
  const int ngrad = ((MASK & 1) ? 1 : 0) + ((MASK & 2) ? 1 : 0);
  char *o1 = ROLE == ROLE_DQ ? p.dq1 : p.dk1;
  char *o2 = ROLE == ROLE_DQ ? p.dq2 : p.dk2;
  const float *part0 = (MASK & 1) ? p.part1 : p.part2;
  char *out0 = (MASK & 1) ? o1 : o2;
  part_reduce_kernel<BF16, ROLE><<<dim3(unsigned(rblocks), unsigned(ngrad)), dim3(256), 0, stream>>>(
      part0, out0, p.part2, o2, p.nsplit, n4 SK_DBG_ARGS(p.part_lo, p.xp, ROLE == ROLE_DQ ? p.xq : p.xk));
  return hipGetLastError();
}

template <int ROLE, bool BF16, int D, bool CAUSAL>
hipError_t launch_bwd_masks(const BwdArgs &a, hipStream_t s) {
  // Only the key-gradient role varies g along a block's rows.
  const bool gsign = ROLE == ROLE_DK && a.dkl != nullptr;
  constexpr bool kDK = ROLE == ROLE_DK && BF16;
  const bool po = kDK && bwd_dk_paired(a.bh, a.nq, a.nk, a.bf16);
  switch (a.grad_mask) {
    case 1: return gsign ? launch_bwd_t<BF16, D, CAUSAL, ROLE, 1, true, false>(a, s)
                         : launch_bwd_t<BF16, D, CAUSAL, ROLE, 1, false, false>(a, s);
    case 2:
      if (po) return gsign ? launch_bwd_t<BF16, D, CAUSAL, ROLE, 2, true, kDK>(a, s)
                           : launch_bwd_t<BF16, D, CAUSAL, ROLE, 2, false, kDK>(a, s);
      return gsign ? launch_bwd_t<BF16, D, CAUSAL, ROLE, 2, true, false>(a, s)
                   : launch_bwd_t<BF16, D, CAUSAL, ROLE, 2, false, false>(a, s);
    default:
      if (po) return gsign ? launch_bwd_t<BF16, D, CAUSAL, ROLE, 3, true, kDK>(a, s)
                           : launch_bwd_t<BF16, D, CAUSAL, ROLE, 3, false, kDK>(a, s);
      return gsign ? launch_bwd_t<BF16, D, CAUSAL, ROLE, 3, true, false>(a, s)
                   : launch_bwd_t<BF16, D, CAUSAL, ROLE, 3, false, false>(a, s);
  }
}

template <int ROLE>
hipError_t launch_bwd_role(const BwdArgs &a, hipStream_t s) {
  if (a.bf16) {
    if (a.d == 64) return a.causal ? launch_bwd_masks<ROLE, true, 64, true>(a, s) : launch_bwd_masks<ROLE, true, 64, false>(a, s);
    return a.causal ? launch_bwd_masks<ROLE, true, 128, true>(a, s) : launch_bwd_masks<ROLE, true, 128, false>(a, s);
  }
  if (a.d == 64) return a.causal ? launch_bwd_masks<ROLE, false, 64, true>(a, s) : launch_bwd_masks<ROLE, false, 64, false>(a, s);
  return a.causal ? launch_bwd_masks<ROLE, false, 128, true>(a, s) : launch_bwd_masks<ROLE, false, 128, false>(a, s);
}

}  // namespace streamkl
