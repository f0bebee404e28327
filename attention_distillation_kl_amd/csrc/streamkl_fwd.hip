// streamkl_fwd.hip -- fused single-pass attention-KL forward kernel (gfx950).
//
// StreamKL summary page (gist.science 2606.20005), "Formulazione Online":
// KL(P1 || P2) of one query row is rewritten in terms of five running row
// scalars -- two shifts m1, m2 for the two logit rows (the page's running
// maxima), the exponential sums l1, l2 taken against them and an accumulator
// acc of the P1-weighted logit difference -- finalised as
// KL = acc / l1 + LSE2 - LSE1, LSE_t = m_t + log l_t.  The page does not print
// the per-tile update.  The rule used here, for a tile of keys J, is
//   l_t = alpha_t l_t + sum_J exp(s_t - m_t'),  alpha_t = exp(m_t - m_t')
//   acc = alpha_1 acc + sum_J exp(s_1 - m_1') (s_1 - s_2)
// which makes acc / l1 = sum_j P1 (s1 - s2) for ANY sequence of shifts; the
// finaliser then equals KL exactly.  The shifts only keep the exponentials in
// range: m_t' = max(m_t, max_J s_t) would do, but computing a maximum per tile
// costs as much as a sum, so a shift is raised only where a tile's sums would
// leave [0, 2^64] (see `pass` and `raise_and_fold` below).
// Key tiles past a query block's causal frontier are never visited.
//
// Mapping to the hardware:
//   * one workgroup = 4 waves x 64 query rows (32 for fp32 with d = 128);
//     each wave keeps its queries' Q1/Q2 fragments in registers for the
//     whole key loop, and every K fragment it reads from LDS feeds the
//     products of both of its 32-query blocks;
//   * K1/K2 tiles (64 keys for bf16, 32 for fp32) are staged in LDS by direct
//     global->LDS copies, double buffered, stored chunk-major;
//   * scores are computed transposed (S^T = K Q^T, 32x32 MFMA blocks) so each
//     lane owns ONE query and 16 keys of every 32-key block: the maxima and
//     sums are in-lane, each lane-half keeps its own five scalars and the two
//     halves are merged once, after the loop (the merge is the same rescale);
//   * exponentials are exp2 with scale*log2(e) folded into one FMA; the
//     shifts are kept on raw dot products and scale is applied at the end;
//   * a wave raises its priority while it issues its matrix products, so the
//     other wave on the SIMD fills the vector unit meanwhile.
#include "streamkl_device.h"
#include "streamkl_launch.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

namespace streamkl {
namespace {

template <bool BF16, int D, bool RM = false>
struct FwdCfg {
  using G = RowGeom<BF16, D>;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  // 32-query blocks per wave; the row-major form (decoding rows) takes one.
  static constexpr int kNQB = RM ? 1 : (BF16 || D == 64) ? 2 : 1;
  static constexpr int kWQ = 32 * kNQB;                   // queries per wave
  static constexpr int kBK = BF16 ? 64 : 32;              // keys per LDS tile
  static constexpr int kSub = kBK / 32;                   // 32-key blocks per tile
  // Waves sharing one query block, each scoring its own 32-key blocks of
  // every tile (the row-major form: decoding rows leave most waves of a
  // workgroup without rows of their own).
  static constexpr int kKSplit = RM ? kSub : 1;
  static constexpr int kBQ = kWQ * kWaves / kKSplit;      // queries per workgroup
  static_assert(kWaves % kKSplit == 0 && kSub % kKSplit == 0, "waves must pair evenly");
  static constexpr int kTileChunks = kBK * G::kChunks;    // 16-B chunks per tensor tile
  static constexpr int kLoads = kTileChunks / kThreads;   // copies per thread per tensor
  static constexpr size_t kLdsBytes = size_t(2) * 2 * kTileChunks * 16;  // 2 stages x K1,K2
  static_assert(kTileChunks % kThreads == 0, "tile must split evenly over the workgroup");
};

struct FwdParams {
  const char *q1, *k1, *q2, *k2;
  float *kl, *lse1, *lse2;
  int nq, nk, nqb;
  float scale, c;  // c = scale * log2(e)
  // Split-K: the key tiles are dealt to nsplit partitions of tps tiles each
  // (causal grids in the rank-major order: each query block's own admissible
  // tiles, in nsplit runs of equal length); partition states go to part =
  // [5][nsplit][bh * nq] (m1, m2, l1, l2, acc).
  int nsplit, tps;
  // Causal: the query blocks' ranks are taken over each XCD's heads (lf 1,
  // unsplit, longest_first) or over the whole grid (lf 2, with partitions)
  // instead of head by head (0).
  int lf;
  size_t rows;  // B * H * N_Q
  float *part;
#ifdef STREAMKL_DEBUG
  size_t xq, xk, xr, xp;  // bytes of a query tensor, a key tensor, a row vector, the partition states
#endif
};

// Row-state layout of the split-K workspace: scalar k of partition s for
// row r (r = bh * N_Q + i) of `rows` rows lives at part[(k * nsplit + s) * rows + r].
enum { ST_M1 = 0, ST_M2, ST_L1, ST_L2, ST_ACC, ST_N };

// RM: key tiles stored row-major with the backward's XOR swizzle instead of
// chunk-major.  Each copy instruction then reads whole key rows (coalesced);
// the fragment reads need one address per chunk.  Used for decoding rows.
// There two waves share each 32-query block, each scoring one of a tile's
// two 32-key blocks, so twice as many waves fold scores; their states are
// merged at the end.
template <bool BF16, int D, bool CAUSAL, bool SPLIT, bool RM = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  using C = FwdCfg<BF16, D, RM>;
  using G = typename C::G;
  constexpr int NQB = C::kNQB;
  extern __shared__ u32x4 lds[];  // [stage][tensor][kTileChunks]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;

  // Heads are contiguous in logical order (one head per XCD at a time); for
  // causal problems the longest query blocks of a head go first, or, with
  // p.lf, the longest of all the XCD's heads (longest_first) or of the whole
  // grid (rank-major, causal grids with partitions).
  // With split-K, the query blocks of one (head, partition) are consecutive,
  // so they share the partition's K tiles in one L2.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_bh = p.nqb * (SPLIT ? p.nsplit : 1);
  int bh = bid / per_bh;
  const int rem = bid - bh * per_bh;
  int split = SPLIT ? rem / p.nqb : 0;
  int qbr = rem - split * p.nqb;
  if (CAUSAL && SPLIT && p.lf == 2) {
    // Rank-major over (rank, head, partition): hardware workgroup b, dealt
    // to the XCDs in turn, so every XCD runs every eighth entry of the list
    // sorted longest first (see rank_major).
    const int per_rank = gridDim.x / p.nqb;
    const int b = blockIdx.x;
    qbr = b / per_rank;
    bh = (b - qbr * per_rank) / p.nsplit;
    split = b - qbr * per_rank - bh * p.nsplit;
  }
  if (CAUSAL && !SPLIT && p.lf) {
    const BlockPos bp = longest_first(bid, gridDim.x, p.nqb);
    bh = bp.bh;
    qbr = bp.rank;
  }
  const int qb = CAUSAL ? p.nqb - 1 - qbr : qbr;
  const int q0 = qb * C::kBQ;
  // The wave's query block and, with kKSplit > 1, which 32-key blocks of a
  // tile it scores (those with sb % kKSplit == ksub).
  const int ksub = wave % C::kKSplit;
  const int wq0 = q0 + (wave / C::kKSplit) * C::kWQ;
  const bool wave_active = wq0 < p.nq;

  const size_t qoff = size_t(bh) * p.nq * G::kRowBytes;
  const size_t koff = size_t(bh) * p.nk * G::kRowBytes;

  // Stationary query fragments (B operand), zero for rows past N_Q.
  u32x4 qf1[NQB][G::kLaneChunks], qf2[NQB][G::kLaneChunks];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int qrow = wq0 + 32 * j + col;
    if (qrow < p.nq) {
      const u32x4 *r1 = reinterpret_cast<const u32x4 *>(p.q1 + qoff + size_t(qrow) * G::kRowBytes);
      const u32x4 *r2 = reinterpret_cast<const u32x4 *>(p.q2 + qoff + size_t(qrow) * G::kRowBytes);
#pragma unroll
      for (int c = 0; c < G::kLaneChunks; ++c) {
        qf1[j][c] = *SK_G((&r1[frag_chunk<BF16, D>(h, c)]), 16, p.q1, p.xq, 1);
        qf2[j][c] = *SK_G((&r2[frag_chunk<BF16, D>(h, c)]), 16, p.q2, p.xq, 1);
      }
    } else {
#pragma unroll
      for (int c = 0; c < G::kLaneChunks; ++c) qf1[j][c] = qf2[j][c] = zero4();
    }
  }

  // Key range: [0, kend).  Causal: the last allowed key of row i is i + N_K - N_Q.
  const int off = p.nk - p.nq;
  int kend = p.nk;
  if (CAUSAL) kend = min(p.nk, min(q0 + C::kBQ, p.nq) + off);
  // Tiles [tile0, tile1) of this workgroup: the partition's share of them.
  int tile0 = 0, tile1 = (kend + C::kBK - 1) / C::kBK;
  if (SPLIT) {
    // Causal grids of more than one round (lf 2): the block's own range in
    // nsplit equal runs, so that all of a block's partitions are about
    // equally long and the rank-major order balances them (a block with
    // fewer tiles than partitions leaves the last ones empty; their states
    // weigh 0).  Within one round every partition runs at once and the
    // longest block's runs are as long either way; there the fixed runs of
    // tps tiles leave fewer workgroups with a tile or two (C2's forward,
    // 8 partitions: 0.041 against 0.042 ms).
    const int len = (CAUSAL && p.lf == 2) ? (tile1 + p.nsplit - 1) / p.nsplit : p.tps;
    tile0 = split * len;
    tile1 = min(tile1, tile0 + len);
  }
  const int ntiles = max(tile1 - tile0, 0);
  // Per 32-query block j of the wave: the lane's last key, and the smallest
  // and largest last key over the block (wave-uniform).
  int my_last[NQB], blk_lo[NQB], blk_hi[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int r0 = wq0 + 32 * j;
    // Without the mask every row ends at the last key: the same formula with
    // offset N_K (in 64 bits) gives N_K - 1.  Writing the constant instead
    // lets the compiler specialise the loop on it, and that instantiation
    // then spills 36 registers.
    const long long eo = CAUSAL ? off : p.nk;
    const long long last = p.nk - 1;
    my_last[j] = int(min((long long)(r0 + col) + eo, last));
    blk_lo[j] = int(min((long long)r0 + eo, last));
    blk_hi[j] = int(min((long long)(r0 + 31) + eo, last));
  }
  const int w_hi = blk_hi[NQB - 1];

  const char *kb1 = p.k1 + koff;
  const char *kb2 = p.k2 + koff;

  // Stage key tile kt into LDS buffer `stage` with direct global->LDS copies.
  // The tile is stored chunk-major: 16-byte chunk c of tile row r sits at
  // position c*kBK + r.  A lane's fragment chunks are then one base address
  // plus compile-time offsets, and the 32 lanes of a half read 32 consecutive
  // chunks (no bank conflicts).  Lane L of wave w fills position
  // i*256 + 64w + L, i.e. reads chunk c of key row r from global memory.
  // Rows past N_K repeat the last key; the compute masks them.
  static_assert(C::kThreads % C::kBK == 0, "a thread copies one tile row");
  const int crow = tid % C::kBK;                // the tile row this thread copies
  const int cch = tid / C::kBK;                 // its first chunk; then every kThreads/kBK
  auto issue = [&](int kt, int stage) {
    if constexpr (RM) {
      // Lane L of wave w fills position i*threads + 64w + L of the row-major
      // tile; the global side reads the (row, logical chunk) stored there.
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        const int pos = i * C::kThreads + tid;
        const int row = pos / G::kChunks;
        const int ch = swz<G::kChunks>(row, pos % G::kChunks);
        const size_t o = size_t(min(kt * C::kBK + row, p.nk - 1)) * G::kRowBytes + ch * 16;
        dma16(SK_G(kb1 + o, 16, p.k1, p.xk, 1),
              SK_L(lds + (stage * 2 + 0) * C::kTileChunks + i * C::kThreads + wave * 64, 1024, lds, C::kLdsBytes, 1));
        dma16(SK_G(kb2 + o, 16, p.k2, p.xk, 1),
              SK_L(lds + (stage * 2 + 1) * C::kTileChunks + i * C::kThreads + wave * 64, 1024, lds, C::kLdsBytes, 1));
      }
      return;
    }
    const int key = min(kt * C::kBK + crow, p.nk - 1);
    const size_t o = size_t(key) * G::kRowBytes + cch * 16;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int oi = i * (C::kThreads / C::kBK) * 16;
      u32x4 *w1 = lds + (stage * 2 + 0) * C::kTileChunks + i * C::kThreads + wave * 64;
      u32x4 *w2 = lds + (stage * 2 + 1) * C::kTileChunks + i * C::kThreads + wave * 64;
      dma16(SK_G(kb1 + o + oi, 16, p.k1, p.xk, 1), SK_L(w1, 1024, lds, C::kLdsBytes, 1));
      dma16(SK_G(kb2 + o + oi, 16, p.k2, p.xk, 1), SK_L(w2, 1024, lds, C::kLdsBytes, 1));
    }
  };

  const float c = p.c;
  // The five running scalars per query block and lane-half.  m1, m2 are the
  // shifts the exponentials are taken against, in raw dot-product units.  They
  // are not re-derived from every block's maximum: they only have to stay at
  // or below the running maximum (so l_t >= 1) and close enough to it that no
  // exponential overflows.  A block whose sums stay within kSumCap (every
  // exponential then lies in [0, 2^64]) is folded as it is; otherwise -- the
  // first admissible block, or logits more than 64 log2-units above the shift
  // -- the lane raises its shifts to the block's maximum, rescales l and acc,
  // and folds the block again.  Any shift yields the same finalised KL and LSE.
  constexpr float kSumCap = 18446744073709551616.f;  // 2^64
  float m1[NQB], m2[NQB], nm1c[NQB], nm2c[NQB], l1[NQB], l2[NQB], acc[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    m1[j] = m2[j] = -INFINITY;
    nm1c[j] = nm2c[j] = INFINITY;  // -m c
    l1[j] = l2[j] = acc[j] = 0.f;
  }

  // Online update of query block j's scalars with one 32-key block of scores:
  // fold against the current shifts; a lane whose sums leave the cap raises
  // its shifts and folds the block again (every term is then <= 1).
  auto pass = [&](int j, const f32x16 &s1, const f32x16 &s2, int kb, auto masked_c) -> bool {
    constexpr bool kMasked = decltype(masked_c)::value;
    // -0 is the additive identity, so the sums start with their first term.
    float ts1a = -0.f, ts1b = -0.f, ts2a = -0.f, ts2b = -0.f, tda = -0.f, tdb = -0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p1a = fast_exp2(fmaf(s1[r], c, nm1c[j]));
      float p2a = fast_exp2(fmaf(s2[r], c, nm2c[j]));
      float p1b = fast_exp2(fmaf(s1[r + 1], c, nm1c[j]));
      float p2b = fast_exp2(fmaf(s2[r + 1], c, nm2c[j]));
      if constexpr (kMasked) {
        const bool oka = kb + c_row(r, h) <= my_last[j];
        const bool okb = kb + c_row(r + 1, h) <= my_last[j];
        p1a = oka ? p1a : 0.f;
        p2a = oka ? p2a : 0.f;
        p1b = okb ? p1b : 0.f;
        p2b = okb ? p2b : 0.f;
      }
      ts1a += p1a;
      ts2a += p2a;
      ts1b += p1b;
      ts2b += p2b;
      tda = fmaf(p1a, s1[r] - s2[r], tda);
      tdb = fmaf(p1b, s1[r + 1] - s2[r + 1], tdb);
    }
    const float ts1 = ts1a + ts1b, ts2 = ts2a + ts2b, td = tda + tdb;
    const bool raise = ts1 > kSumCap || ts2 > kSumCap;
    // Selects rather than a branch: the terms are consumed as they are made.
    l1[j] += raise ? 0.f : ts1;
    l2[j] += raise ? 0.f : ts2;
    acc[j] += raise ? 0.f : td;
    return raise;
  };
  // Scores of query block j alone against the 32 keys at tile row sb*32 of
  // buffers (kb1s, kb2s): used where a block has to be folded again.
  auto rescore = [&](int j, int sb, const u32x4 *t1, const u32x4 *t2, f32x16 &s1, f32x16 &s2) {
    s1 = f32x16{};
    s2 = f32x16{};
    const int row = sb * 32 + col;
#pragma unroll
    for (int cc = 0; cc < G::kLaneChunks; ++cc) {
      const int pos = RM ? row * G::kChunks + swz<G::kChunks>(row, frag_chunk<BF16, D>(h, cc))
                         : frag_chunk<BF16, D>(h, cc) * C::kBK + row;
      mfma_chunk<BF16>(*SK_L(&t1[pos], 16, lds, C::kLdsBytes, 1), qf1[j][cc], s1);
      mfma_chunk<BF16>(*SK_L(&t2[pos], 16, lds, C::kLdsBytes, 1), qf2[j][cc], s2);
    }
  };
  // A raise (rare: the first admissible block of a row, or an overflow)
  // happens after every query block's first pass, when no score register is
  // live any more: the scores are recomputed from the tile, still in LDS.
  auto raise_and_fold = [&](int j, const f32x16 &r1, const f32x16 &r2, int kb) {
    float u1 = m1[j], u2 = m2[j];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = kb + c_row(r, h) <= my_last[j];
      u1 = vmax(u1, ok ? r1[r] : -INFINITY);
      u2 = vmax(u2, ok ? r2[r] : -INFINITY);
    }
    const float a1 = (m1[j] == -INFINITY) ? 0.f : fast_exp2((m1[j] - u1) * c);
    const float a2 = (m2[j] == -INFINITY) ? 0.f : fast_exp2((m2[j] - u2) * c);
    l1[j] *= a1;
    acc[j] *= a1;
    l2[j] *= a2;
    m1[j] = u1;
    m2[j] = u2;
    nm1c[j] = -u1 * c;
    nm2c[j] = -u2 * c;
    pass(j, r1, r2, kb, std::true_type{});
  };

  if (ntiles > 0) issue(tile0, 0);
  __syncthreads();

  for (int kt = tile0; kt < tile1; ++kt) {
    const int stage = (kt - tile0) & 1;
    // Buffer stage^1 was last read in iteration kt-1, which ended in a barrier.
    if (kt + 1 < tile1) issue(kt + 1, stage ^ 1);
    const u32x4 *b1 = lds + (stage * 2 + 0) * C::kTileChunks;
    const u32x4 *b2 = lds + (stage * 2 + 1) * C::kTileChunks;

#pragma unroll
    for (int sb = 0; sb < C::kSub; ++sb) {
      if (C::kKSplit > 1 && sb % C::kKSplit != ksub) continue;  // another wave's keys
      const int kb = kt * C::kBK + sb * 32;
      if (!wave_active || kb > w_hi) continue;  // past every row's frontier

      // Scores S^T = K Q^T of this key block for all query blocks: each K
      // fragment is read from LDS once and used for NQB products.
      f32x16 s1[NQB], s2[NQB];
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        s1[j] = f32x16{};
        s2[j] = f32x16{};
      }
      const int row = sb * 32 + col;
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int cc = 0; cc < G::kLaneChunks; ++cc) {
        const int pos = RM ? row * G::kChunks + swz<G::kChunks>(row, frag_chunk<BF16, D>(h, cc))
                           : frag_chunk<BF16, D>(h, cc) * C::kBK + row;
        const u32x4 a1 = *SK_L(&b1[pos], 16, lds, C::kLdsBytes, 1), a2 = *SK_L(&b2[pos], 16, lds, C::kLdsBytes, 1);
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          mfma_chunk<BF16>(a1, qf1[j][cc], s1[j]);
          mfma_chunk<BF16>(a2, qf2[j][cc], s2[j]);
        }
      }
      if constexpr (BF16) {
        // Keep each K fragment read next to its products: reading all of them
        // up front would need 64 more registers than a wave has.
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // 2 LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NQB, 0);  // their products
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);

      // Fold each query block: plain when the whole block is admissible.
      bool plain = true, rz[NQB];
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        plain = plain && kb + 31 <= blk_lo[j];
        rz[j] = false;
      }
      if (plain) {
#pragma unroll
        for (int j = 0; j < NQB; ++j) rz[j] = pass(j, s1[j], s2[j], kb, std::false_type{});
      } else {
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          if (kb > blk_hi[j]) continue;
          if (kb + 31 > blk_lo[j]) rz[j] = pass(j, s1[j], s2[j], kb, std::true_type{});
          else rz[j] = pass(j, s1[j], s2[j], kb, std::false_type{});
        }
      }
      bool any = false;
#pragma unroll
      for (int j = 0; j < NQB; ++j) any = any || rz[j];
      // Wave-uniform branches: the products of a recompute need every lane.
      if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          if (__builtin_amdgcn_ballot_w64(rz[j]) == 0) continue;
          f32x16 r1, r2;
          rescore(j, sb, b1, b2, r1, r2);
          if (rz[j]) raise_and_fold(j, r1, r2, kb);
        }
      }
    }
    __syncthreads();  // also waits for the copies into stage^1
  }

  // Merge the two lane-halves (disjoint key subsets of the same query).
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const float om1 = __shfl_xor(m1[j], 32), om2 = __shfl_xor(m2[j], 32);
    const float ol1 = __shfl_xor(l1[j], 32), ol2 = __shfl_xor(l2[j], 32);
    const float oacc = __shfl_xor(acc[j], 32);
    float M1 = vmax(m1[j], om1), M2 = vmax(m2[j], om2);
    const float fa1 = (m1[j] == -INFINITY) ? 0.f : fast_exp2((m1[j] - M1) * c);
    const float fb1 = (om1 == -INFINITY) ? 0.f : fast_exp2((om1 - M1) * c);
    const float fa2 = (m2[j] == -INFINITY) ? 0.f : fast_exp2((m2[j] - M2) * c);
    const float fb2 = (om2 == -INFINITY) ? 0.f : fast_exp2((om2 - M2) * c);
    float L1 = l1[j] * fa1 + ol1 * fb1;
    float L2 = l2[j] * fa2 + ol2 * fb2;
    float A = acc[j] * fa1 + oacc * fb1;
    if constexpr (C::kKSplit > 1) {
      // Merge the waves that scored disjoint key blocks of the same rows, the
      // same way, through LDS: the tile buffers are free, since the loop
      // ended in a barrier after its last reads and no copy is in flight.
      static_assert(C::kKSplit == 2 && NQB == 1, "one partner wave, one query block");
      float *x = SK_L(reinterpret_cast<float *>(lds) + (wave / 2) * (ST_N * 32) + col, ((ST_N - 1) * 32 + 1) * 4,
                      lds, C::kLdsBytes, 1);
      __syncthreads();
      if (ksub == 1 && h == 0) {
        x[ST_M1 * 32] = M1;
        x[ST_M2 * 32] = M2;
        x[ST_L1 * 32] = L1;
        x[ST_L2 * 32] = L2;
        x[ST_ACC * 32] = A;
      }
      __syncthreads();
      if (ksub == 1) continue;  // the even wave of the pair writes the rows
      const float pm1 = x[ST_M1 * 32], pm2 = x[ST_M2 * 32];
      const float N1 = vmax(M1, pm1), N2 = vmax(M2, pm2);
      const float ga1 = (M1 == -INFINITY) ? 0.f : fast_exp2((M1 - N1) * c);
      const float gb1 = (pm1 == -INFINITY) ? 0.f : fast_exp2((pm1 - N1) * c);
      const float ga2 = (M2 == -INFINITY) ? 0.f : fast_exp2((M2 - N2) * c);
      const float gb2 = (pm2 == -INFINITY) ? 0.f : fast_exp2((pm2 - N2) * c);
      L1 = L1 * ga1 + x[ST_L1 * 32] * gb1;
      L2 = L2 * ga2 + x[ST_L2 * 32] * gb2;
      A = A * ga1 + x[ST_ACC * 32] * gb1;
      M1 = N1;
      M2 = N2;
    }
    const int qrow = wq0 + 32 * j + col;
    if (SPLIT) {
      // The partition's state, merged with the others by merge_kernel.
      if (h == 0 && qrow < p.nq) {
        const size_t r = size_t(bh) * p.nq + qrow;
        float *out = p.part + size_t(split) * p.rows + r;
        const size_t stride = size_t(p.nsplit) * p.rows;
        auto put = [&](float *q, float v) {
          if (SK_OK(q, 4, p.part, p.xp, 1)) *q = v;
        };
        put(out + ST_M1 * stride, M1);
        put(out + ST_M2 * stride, M2);
        put(out + ST_L1 * stride, L1);
        put(out + ST_L2 * stride, L2);
        put(out + ST_ACC * stride, A);
      }
      continue;
    }
    if (h == 0 && qrow < p.nq) {
      const float lse1 = M1 * p.scale + logf(L1);
      const float lse2 = M2 * p.scale + logf(L2);
      const size_t o = size_t(bh) * p.nq + qrow;
      if (SK_OK(p.kl + o, 4, p.kl, p.xr, 1)) p.kl[o] = p.scale * (A / L1) + lse2 - lse1;
      if (SK_OK(p.lse1 + o, 4, p.lse1, p.xr, 1)) p.lse1[o] = lse1;
      if (SK_OK(p.lse2 + o, 4, p.lse2, p.xr, 1)) p.lse2[o] = lse2;
    }
  }
}

// Split-K merge.  A row's partition states are combined with the rescale of
// the online update (empty partitions, m = -inf, weigh 0) and the row is then
// finalised as the unsplit kernel does.  G = min(64, next power of two >=
// nsplit) consecutive lanes take one row: lane j reads partitions j, j + G,
// ..., so that a row's loads are in flight together rather than one
// partition after another, and the lanes' states are then combined pairwise
// across the group.  With one partition the row's state is finalised as
// stored, which reproduces the unsplit results bit for bit.
struct RowState {
  float m1, m2, l1, l2, acc;
};
__device__ __forceinline__ RowState combine(const RowState &a, const RowState &b, float c) {
  RowState r;
  r.m1 = vmax(a.m1, b.m1);
  r.m2 = vmax(a.m2, b.m2);
  const float fa1 = (a.m1 == -INFINITY) ? 0.f : fast_exp2((a.m1 - r.m1) * c);
  const float fb1 = (b.m1 == -INFINITY) ? 0.f : fast_exp2((b.m1 - r.m1) * c);
  const float fa2 = (a.m2 == -INFINITY) ? 0.f : fast_exp2((a.m2 - r.m2) * c);
  const float fb2 = (b.m2 == -INFINITY) ? 0.f : fast_exp2((b.m2 - r.m2) * c);
  r.l1 = fmaf(a.l1, fa1, b.l1 * fb1);
  r.l2 = fmaf(a.l2, fa2, b.l2 * fb2);
  r.acc = fmaf(a.acc, fa1, b.acc * fb1);
  return r;
}

template <int G>
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ part, int nsplit, size_t rows,
                                                    float scale, float c, float *kl, float *lse1,
                                                    float *lse2 SK_DBG_ARGS(size_t xp, size_t xr)) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "a row's lanes lie in one wave");
  const size_t t = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t r = t / G;
  const int j = int(t % G);
  // No early exit: every lane of a group takes part in the exchanges below
  // (a group is wholly inside or wholly past the last row).
  const bool live = r < rows;
  const size_t stride = size_t(nsplit) * rows;
  RowState s{-INFINITY, -INFINITY, 0.f, 0.f, 0.f};
  if (live) {
    for (int k = j; k < nsplit; k += G) {
      const float *st = part + size_t(k) * rows + r;
      const RowState x{*SK_G(&st[ST_M1 * stride], 4, part, xp, 1), *SK_G(&st[ST_M2 * stride], 4, part, xp, 1),
                       *SK_G(&st[ST_L1 * stride], 4, part, xp, 1), *SK_G(&st[ST_L2 * stride], 4, part, xp, 1),
                       *SK_G(&st[ST_ACC * stride], 4, part, xp, 1)};
      s = (k == j) ? x : combine(s, x, c);
    }
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    const RowState y{__shfl_xor(s.m1, o), __shfl_xor(s.m2, o), __shfl_xor(s.l1, o), __shfl_xor(s.l2, o),
                     __shfl_xor(s.acc, o)};
    s = combine(s, y, c);
  }
  if (live && j == 0) {
    const float l1 = s.m1 * scale + logf(s.l1);
    const float l2 = s.m2 * scale + logf(s.l2);
    if (SK_OK(kl + r, 4, kl, xr, 1)) kl[r] = scale * (s.acc / s.l1) + l2 - l1;
    if (SK_OK(lse1 + r, 4, lse1, xr, 1)) lse1[r] = l1;
    if (SK_OK(lse2 + r, 4, lse2, xr, 1)) lse2[r] = l2;
  }
}

// Launches the merge with the smallest lane group that holds nsplit
// partitions (at most 64 lanes; more partitions are looped over).
inline hipError_t launch_merge(const float *part, int nsplit, size_t rows, float scale, float c, float *kl,
                               float *lse1, float *lse2, hipStream_t stream) {
#ifdef STREAMKL_DEBUG
  const size_t xp = size_t(ST_N) * nsplit * rows * sizeof(float), xr = rows * sizeof(float);
#endif
  int g = 1;
  while (g < nsplit && g < 64) g *= 2;
  const size_t threads = rows * size_t(g);
  const size_t blocks = (threads + 255) / 256;
  if (blocks > size_t(INT_MAX)) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks)}, block{256u};
  switch (g) {
    case 1: merge_kernel<1><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    case 2: merge_kernel<2><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    case 4: merge_kernel<4><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    case 8: merge_kernel<8><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    case 16: merge_kernel<16><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    case 32: merge_kernel<32><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
    default: merge_kernel<64><<<grid, block, 0, stream>>>(part, nsplit, rows, scale, c, kl, lse1, lse2 SK_DBG_ARGS(xp, xr)); break;
  }
  return hipGetLastError();
}

// Whether the causal, unsplit forward takes its query blocks' ranks over each
// XCD's heads (longest_first_pays, with two resident workgroups per CU and 32
// CUs per XCD).  Measured at 64 heads x 32 query blocks: -11%; at 128 blocks
// a head, where it would not help, the shared L2 made it 2-4% slower.
inline bool fwd_longest_first(long long nwg, long long nqb) { return longest_first_pays(nwg, nqb, 2 * 32); }

template <bool BF16, int D, bool CAUSAL, bool RM = false>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
  using C = FwdCfg<BF16, D, RM>;
  FwdParams p;
  p.q1 = static_cast<const char *>(a.q1);
  p.k1 = static_cast<const char *>(a.k1);
  p.q2 = static_cast<const char *>(a.q2);
  p.k2 = static_cast<const char *>(a.k2);
  p.kl = a.kl;
  p.lse1 = a.lse1;
  p.lse2 = a.lse2;
  p.nq = a.nq;
  p.nk = a.nk;
  p.nqb = (a.nq + C::kBQ - 1) / C::kBQ;
  p.scale = a.scale;
  p.c = float(double(a.scale) * 1.4426950408889634);
  p.rows = size_t(a.bh) * a.nq;
  const bool split = a.splits > 1;
  const int total_tiles = (a.nk + C::kBK - 1) / C::kBK;
  p.nsplit = split ? a.splits : 1;
  p.tps = (total_tiles + p.nsplit - 1) / p.nsplit;
  p.part = a.part;
#ifdef STREAMKL_DEBUG
  p.xq = size_t(a.bh) * a.nq * C::G::kRowBytes;
  p.xk = size_t(a.bh) * a.nk * C::G::kRowBytes;
  p.xr = size_t(a.bh) * a.nq * sizeof(float);
  p.xp = split ? size_t(ST_N) * p.nsplit * p.rows * sizeof(float) : 0;
#endif
  // Causal grids with partitions of more than one round (two workgroups per
  // CU) take the rank-major order: the partitions of a head's long blocks
  // then spread over every XCD.
  p.lf = !CAUSAL ? 0
         : split ? ((long long)p.nqb * a.bh * p.nsplit > 2 * 256 ? 2 : 0)
                 : (fwd_longest_first((long long)p.nqb * a.bh, p.nqb) ? 1 : 0);
  const long long blocks = (long long)p.nqb * a.bh * p.nsplit;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  void *args[] = {&p};
  const void *fn = split ? reinterpret_cast<const void *>(&fwd_kernel<BF16, D, CAUSAL, true, RM>)
                         : reinterpret_cast<const void *>(&fwd_kernel<BF16, D, CAUSAL, false, RM>);
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(C::kThreads), args, C::kLdsBytes, stream);
  if (e != hipSuccess || !split) return e;
  return launch_merge(a.part, p.nsplit, p.rows, p.scale, p.c, a.kl, a.lse1, a.lse2, stream);
}

}  // namespace

int fwd_default_splits(int bh, int nq, int nk, int d, bool bf16, bool causal) {
  // Partitions of the key dimension so that the grid fills one round of
  // resident workgroups (two per CU), each partition keeping at least four
  // key tiles.  (Measured: a second round of half-size partitions costs up
  // to 20% more for short query blocks, since each workgroup also pays its
  // fragment loads and state stores.)  Causal problems with N_Q > N_K / 2
  // are uneven: the causal triangle makes the query blocks' work differ up
  // to N_Q / 256 fold.  Over more than one round, the unsplit kernel
  // balances them by taking the longest blocks of each XCD's heads first,
  // where it can (fwd_longest_first; measured 0.58 ms unsplit against 0.70
  // in two partitions at 32 heads x 8K tokens, 0.30 against 0.38 at 64 x
  // 4K).  Within one round, or where it cannot, they get partitions of at
  // least 16 tiles for about four rounds, which lets the workgroups balance
  // (measured 5-17% faster at 4K-8K tokens than one partition taken head by
  // head; 0.23 against 0.24 ms at 32 x 4K with the blocks sorted).  The
  // larger of the two counts is taken.
  const bool nqb2 = bf16 || d == 64;
  const int kbq = nqb2 ? 256 : 128, kbk = bf16 ? 64 : 32;
  const long long nqb = (nq + kbq - 1) / kbq;
  const long long nwg = (long long)bh * nqb;
  if (nwg <= 0) return 1;
  const long long tiles = (nk + kbk - 1) / kbk;
  auto count = [&](long long target, long long min_tiles) {
    if (nwg >= target) return 1LL;
    return std::min((target + nwg - 1) / nwg, std::max(1LL, tiles / min_tiles));
  };
  long long s = count(2 * 256, 4);
  if (causal && 2LL * nq > nk && (nwg <= 2 * 256 || !fwd_longest_first(nwg, nqb)))
    s = std::max(s, count(8 * 256, 16));
  return int(std::min(s, 256LL));
}

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
  // Decoding rows (key partitions whose query rows fit one wave): row-major
  // key tiles, whose copies read whole rows.
  if (a.bf16 && a.splits > 1 && a.nq <= FwdCfg<true, 128>::kWQ) {
    if (a.d == 64) return a.causal ? launch<true, 64, true, true>(a, stream) : launch<true, 64, false, true>(a, stream);
    return a.causal ? launch<true, 128, true, true>(a, stream) : launch<true, 128, false, true>(a, stream);
  }
  if (a.bf16) {
    if (a.d == 64) return a.causal ? launch<true, 64, true>(a, stream) : launch<true, 64, false>(a, stream);
    return a.causal ? launch<true, 128, true>(a, stream) : launch<true, 128, false>(a, stream);
  }
  if (a.d == 64) return a.causal ? launch<false, 64, true>(a, stream) : launch<false, 64, false>(a, stream);
  return a.causal ? launch<false, 128, true>(a, stream) : launch<false, 128, false>(a, stream);
}

#ifdef STREAMKL_DEBUG
unsigned dbg_take_fwd() { return dbg_take(); }
#endif
}  // namespace streamkl
