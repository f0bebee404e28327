// streamkl_bwd_fused.hip -- single-pass recompute backward with query
// gradients added by atomics (gfx950, bf16 inputs).
//
// StreamKL summary page (gist.science 2606.20005), "Strategia di Ricalcolo",
// kernel-fusion bullet: the backward visits each (query tile, key tile) pair
// once, keeping dK in registers and adding dQ into a buffer with atomic adds
// while that buffer fits in L2; where it does not, two separate kernels are
// used (the separate-kernel form lives in streamkl_bwd.h).  "Risultati
// Sperimentali", ablation bullet: the fused form pays off for short query
// blocks.  The arithmetic is the recompute of the separate-kernel form:
//   P1 = exp2(s1' c), s1' = s1 - LSE1/scale;   s2'' = s2 + (KL - LSE2)/scale
//   P2 = exp2(s2'' c - KL c/scale)
//   e2 = g (P2 - P1)                    (dS2 = e2)
//   e1 = g P1 (s1' - s2'')              (dS1 = scale e1)
//   dK_t = f_t e_t^T Q_t,  dQ_t = f_t e_t K_t,  f1 = scale^2, f2 = scale
// with s_t the raw dot products and c = scale log2(e).
//
// Mapping:
//   * a workgroup owns 128 key rows, one wave per 32 ("stationary"), and
//     streams 64-row query tiles from its causal frontier to N_Q through LDS
//     (direct global->LDS copies, double buffered, XOR-swizzled rows);
//   * per 32-query block each wave recomputes S1^T, S2^T for its keys
//     (queries from LDS as A operand, its keys in registers as B operand: a
//     lane owns one key and 16 queries), forms e1, e2, adds dK_t^T += Q_t^T e_t
//     (Q_t^T by transposing LDS reads), and stores e_t as bf16 into an LDS
//     buffer laid out [key][query];
//   * after a barrier, wave w forms dQ_t for one 32-column slice of d
//     (mb = w % (d/32)) over the keys of its key group (all 128 at d = 128,
//     64 at d = 64): dQ_t block (32 queries x 32 columns) = e_t (from the
//     buffer, transposing reads) x K_t (fragments read once from the
//     stationary tile at the start).  The sum over the workgroup's keys is
//     thus formed on the matrix cores, and each lane adds 16 values per block
//     and gradient with fp32 atomics; for one register the 64 lanes cover 32
//     consecutive columns of two rows, i.e. two 128-byte lines;
//   * the fp32 buffer is zeroed by a fill kernel before and converted to the
//     gradient's element type (times f_t) by a second kernel after.
// With one query tile per head (N_Q <= 64, the sizes streamkl_bwd sends
// here) the kernel takes a second form, which turns the per-block chain of
// copy, barrier, products and atomics into a pipeline:
//   * a workgroup loads the query tile and its row constants once and walks
//     up to 64 consecutive key blocks; each block's stationary tiles are
//     copied (out of the compiler's sight, waited for explicitly) while the
//     previous block is worked on;
//   * the e values stay packed in registers after the scores, and dK is
//     formed one 32-column slice of d at a time, each slice stored as soon
//     as it is complete: 32 accumulator registers instead of 128;
//   * which leaves room to sum each wave's dQ blocks over all of the
//     workgroup's key blocks in registers: one round of atomics per
//     workgroup instead of one per key block.
// The order of the atomic additions varies from run to run, so dQ is not
// bitwise reproducible (dK is).
#include "streamkl_device.h"
#include "streamkl_launch.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

namespace streamkl {
namespace {

template <int D>
struct FusedCfg {
  using G = RowGeom<true, D>;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBS = 32 * kWaves;                  // stationary keys per workgroup
  static constexpr int kBT = 64;                           // streamed queries per tile
  static constexpr int kSub = kBT / 32;                    // 32-query blocks per tile
  static constexpr int kMB = D / 32;                       // 32-column slices of d
  static constexpr int kGroups = kWaves / kMB;             // key groups of the dQ products
  static constexpr int kGroupKeys = kBS / kGroups;         // keys per group: 128 (d = 128), 64 (d = 64)
  static constexpr int kKSteps = kGroupKeys / 16;          // 16-key steps of a dQ product
  static constexpr int kTileChunks = kBT * G::kChunks;     // 16-byte chunks per query tile and tensor
  static constexpr int kLoads = kTileChunks / kThreads;    // copies per thread per tensor
  static constexpr int kXChunks = kBS * G::kChunks;        // stationary tile, per tensor
  static constexpr int kXLoads = kXChunks / kThreads;
  static constexpr int kERowBytes = kBT * 2;               // one key's e row: 64 bf16
  static constexpr int kEBytes = kBS * kERowBytes;         // e buffer, per tensor
  // LDS (bytes): row constants of both stages, two query stages (Q1, Q2),
  // the e buffers (e1, e2).  The stationary tiles (K1, K2) are needed only
  // at the start; they share the space of stage 1 and the e buffers.
  static constexpr int kCstBytes = 2 * 4 * kBT * 4;
  static constexpr int kStageBytes = 2 * kTileChunks * 16;
  static constexpr int kOffStage0 = kCstBytes;
  static constexpr int kOffStage1 = kOffStage0 + kStageBytes;
  static constexpr int kOffE = kOffStage1 + kStageBytes;
  static constexpr int kOffX = kOffStage1;
  static constexpr int kLdsBytes = kOffE + 2 * kEBytes;
  static_assert(kOffX + 2 * kXChunks * 16 <= kLdsBytes, "stationary tiles must fit the shared space");
  // One query tile for the whole workgroup (N_Q <= kBT), which walks several
  // key blocks: no second query stage; the e buffers take its place and the
  // stationary tiles get space of their own, so that the next block's copies
  // overlap the current block's work.
  static constexpr int kOffEM = kOffStage1;
  static constexpr int kOffXM = kOffEM + 2 * kEBytes;
  static constexpr int kLdsBytesM = kOffXM + 2 * kXChunks * 16;
  static_assert(kLdsBytesM <= 160 * 1024, "LDS budget");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  static_assert(kTileChunks % kThreads == 0 && kXChunks % kThreads == 0, "tiles split evenly");
  static_assert(kWaves % kMB == 0, "d slices split the waves evenly");
};

struct FusedParams {
  const char *q1, *k1, *q2, *k2;
  const float *kl, *lse1, *lse2, *dkl;
  char *dk1, *dk2;
  float *ws1, *ws2;   // fp32 query-gradient sums [bh][N_Q][d], zero on entry
  int nq, nk, nsb;    // nsb: stationary blocks per head
  int kbpw;           // key blocks per workgroup (the one-tile form; 1 otherwise)
  float scale, c, inv_scale;
#ifdef STREAMKL_DEBUG
  size_t xq, xk, xr, xw;  // bytes of a query tensor, a key tensor, a row vector, one gradient's sums
#endif
};

// Byte offset of (key, query) in an e buffer: rows of 64 bf16, 16-byte
// chunks XOR-swizzled by the key's low three bits.  A transposing read takes
// 4 consecutive queries (8 bytes, inside one chunk) from each of 8 keys, and
// a store writes 4 consecutive queries for 32 keys: both spread over all
// banks.
__device__ __forceinline__ int ebyte(int key, int q) {
  return key * 128 + (((q >> 3) ^ (key & 7)) << 4) + (q & 7) * 2;
}

template <int D, bool CAUSAL, int MASK, bool GSIGN, bool MULTI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fused_bwd_kernel(FusedParams p) {
  using C = FusedCfg<D>;
  using G = typename C::G;
  constexpr bool kG1 = (MASK & 1) != 0;
  constexpr bool kG2 = (MASK & 2) != 0;
  constexpr int kMB = C::kMB;
  extern __shared__ u32x4 lds[];
  char *lbase = reinterpret_cast<char *>(lds);
  float (*cstage)[4 * C::kBT] = reinterpret_cast<float (*)[4 * C::kBT]>(lbase);
  u32x4 *ystage0 = reinterpret_cast<u32x4 *>(lbase + C::kOffStage0);
  u32x4 *ystage1 = reinterpret_cast<u32x4 *>(lbase + C::kOffStage1);
  char *ebuf = lbase + (MULTI ? C::kOffEM : C::kOffE);  // [tensor][key][query] bf16, swizzled
  u32x4 *xtile = reinterpret_cast<u32x4 *>(lbase + (MULTI ? C::kOffXM : C::kOffX));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int s16 = lane & 15, grp = lane >> 4;
#ifdef STREAMKL_DEBUG
  constexpr size_t kDyn = MULTI ? C::kLdsBytesM : C::kLdsBytes;
#endif

  // Workgroup g of a head takes key blocks [g kbpw, min((g + 1) kbpw, nsb)),
  // key block 0 first: with the mask it sees the most queries.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int kbpw = MULTI ? p.kbpw : 1;
  const int ngrp = (p.nsb + kbpw - 1) / kbpw;
  const int bh = bid / ngrp;
  const int blk0 = (bid - bh * ngrp) * kbpw;
  const int blk1 = min(blk0 + kbpw, p.nsb);
  const int off = p.nk - p.nq;

  const size_t koff = size_t(bh) * p.nk * G::kRowBytes;
  const char *Y1 = p.q1 + size_t(bh) * p.nq * G::kRowBytes;
  const char *Y2 = p.q2 + size_t(bh) * p.nq * G::kRowBytes;

  // The wave's keys in key block kb: the first one (w0), the lane's (srow),
  // its first admissible query (lim), and whether any of the wave's keys is
  // past N_K (wave-uniform).
  struct Blk {
    int s0, w0, srow, lim;
    bool keys_past_end;
  };
  auto blk_state = [&](int kb) {
    Blk b;
    b.s0 = kb * C::kBS;
    b.w0 = b.s0 + wave * 32;
    b.srow = b.w0 + col;
    b.lim = CAUSAL ? max(b.srow - off, 0) : 0;
    b.keys_past_end = b.w0 + 31 >= p.nk;
    return b;
  };

  // Stationary key tiles of block kb -> LDS (rows past N_K repeat the last
  // one; their e values are zero).  The score products' key fragments and
  // the dQ products' key columns are both read from them, so each key row
  // is fetched from memory once.
  // `unseen`: copies issued out of the compiler's sight (dma16_unseen); the
  // caller waits for them (vmcnt0_wait) before the barrier that publishes
  // the tiles.
  auto load_x = [&](int kb, auto unseen_c) {
    const int s0 = kb * C::kBS;
    const char *K1 = p.k1 + koff + size_t(s0) * G::kRowBytes;
    const char *K2 = p.k2 + koff + size_t(s0) * G::kRowBytes;
#pragma unroll
    for (int i = 0; i < C::kXLoads; ++i) {
      const int pos = i * C::kThreads + tid;
      const int row = pos / G::kChunks;
      const int ch = swz<G::kChunks>(row, pos % G::kChunks);
      const uint32_t o = uint32_t(min(s0 + row, p.nk - 1) - s0) * G::kRowBytes + ch * 16;
#ifdef STREAMKL_DEBUG
      // Checked copies go through the builtin; the unseen form's waits stay.
      dma16(SK_G(K1 + o, 16, p.k1, p.xk, 3), SK_L(xtile + i * C::kThreads + wave * 64, 1024, lds, kDyn, 3));
      dma16(SK_G(K2 + o, 16, p.k2, p.xk, 3),
            SK_L(xtile + C::kXChunks + i * C::kThreads + wave * 64, 1024, lds, kDyn, 3));
#else
      if constexpr (decltype(unseen_c)::value) {
        dma16_unseen(K1, o, xtile + i * C::kThreads + wave * 64);
        dma16_unseen(K2, o, xtile + C::kXChunks + i * C::kThreads + wave * 64);
      } else {
        dma16(K1 + o, xtile + i * C::kThreads + wave * 64);
        dma16(K2 + o, xtile + C::kXChunks + i * C::kThreads + wave * 64);
      }
#endif
    }
  };

  auto issue = [&](int tile, int stage) {
    u32x4 *wbase = (stage ? ystage1 : ystage0) + wave * 64;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int pos = i * C::kThreads + tid;
      const int row = pos / G::kChunks;
      const int ch = swz<G::kChunks>(row, pos % G::kChunks);
      const size_t o = size_t(min(tile * C::kBT + row, p.nq - 1)) * G::kRowBytes + ch * 16;
      dma16(SK_G(Y1 + o, 16, p.q1, p.xq, 3), SK_L(wbase + i * C::kThreads, 1024, lds, kDyn, 3));
      dma16(SK_G(Y2 + o, 16, p.q2, p.xq, 3), SK_L(wbase + i * C::kThreads + C::kTileChunks, 1024, lds, kDyn, 3));
    }
  };
  // Per-row constants of a query tile (see the header comment), written by
  // the first 64 threads into the stage's constant arrays.
  auto cwrite = [&](int tile, int stage) {
    if (tid < C::kBT) {
      const int row = tile * C::kBT + tid;
      float *cst = SK_L(cstage[stage], 4 * C::kBT * 4, lds, kDyn, 3);
      if (row < p.nq) {
        const size_t i = size_t(bh) * p.nq + row;
        const float lse1 = *SK_G(&p.lse1[i], 4, p.lse1, p.xr, 3), lse2 = *SK_G(&p.lse2[i], 4, p.lse2, p.xr, 3);
        const float kl = *SK_G(&p.kl[i], 4, p.kl, p.xr, 3);
        cst[tid] = -lse1 * p.inv_scale;
        cst[C::kBT + tid] = (kl - lse2) * p.inv_scale;
        cst[2 * C::kBT + tid] = p.dkl ? *SK_G(&p.dkl[i], 4, p.dkl, p.xr, 3) : 1.f;
        cst[3 * C::kBT + tid] = -kl * p.inv_scale * p.c;
      } else {  // rows past N_Q: P = 0 and s1' - s2'' = 0
        cst[tid] = -1e30f;
        cst[C::kBT + tid] = -1e30f;
        cst[2 * C::kBT + tid] = 0.f;
        cst[3 * C::kBT + tid] = 0.f;
      }
    }
  };

  // Key fragments of the score products (B operand: lane = key, the chunks
  // of its half of d) and the K_t fragments of the dQ products (B operand:
  // lane = column of d, 8 keys per half), read from the stationary tiles
  // (transposing reads for the latter).  Key order within a 16-key step:
  // position 4t + j holds key 16 ks + 8 t + 4 h + j, the order the e buffer
  // reads below use as well.  A key past N_K reads the repeated last row;
  // its scores are masked.
  const int mb = wave % kMB;
  const int kg = wave / kMB;
  u32x4 xf1[G::kLaneChunks], xf2[G::kLaneChunks];
  u32x4 kt1[C::kKSteps], kt2[C::kKSteps];
  auto read_frags = [&]() {
    const int xrow = wave * 32 + col;
#pragma unroll
    for (int cc = 0; cc < G::kLaneChunks; ++cc) {
      const int pos = xrow * G::kChunks + swz<G::kChunks>(xrow, frag_chunk<true, D>(h, cc));
      xf1[cc] = *SK_L(&xtile[pos], 16, lds, kDyn, 3);
      xf2[cc] = *SK_L(&xtile[C::kXChunks + pos], 16, lds, kDyn, 3);
    }
    const int d0 = mb * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = kg * C::kGroupKeys + 16 * ks + 8 * t + 4 * h + (s16 >> 2);
        const int byte = (row * G::kChunks + swz<G::kChunks>(row, d0 >> 3)) * 16 + (d0 & 7) * 2;
        if (kG1) {
          const u32x2 v = read_tr(SK_L(reinterpret_cast<const char *>(xtile) + byte, 8, lds, kDyn, 3));
          kt1[ks][2 * t] = v[0];
          kt1[ks][2 * t + 1] = v[1];
        }
        if (kG2) {
          const u32x2 v = read_tr(SK_L(reinterpret_cast<const char *>(xtile + C::kXChunks) + byte, 8, lds, kDyn, 3));
          kt2[ks][2 * t] = v[0];
          kt2[ks][2 * t + 1] = v[1];
        }
      }
    }
  };

  f32x16 acc1[kMB], acc2[kMB];
  const float c = p.c;

  // Steps 1-4 for the query tile `tile` (in LDS stage `stage`) and the keys
  // of block B: scores, e values, dK_t^T += Q_t^T e_t, e values to the
  // buffer.  Without `grad_c` step 3 is left out and the packed e values
  // are kept in `pks` [32-query block][tensor][16-query step] instead.
  using PackedE = u32x4[C::kSub][2][2];
  auto tile_work = [&](int tile, int stage, const Blk &B, auto grad_c, PackedE &pks) {
    constexpr bool kInlineGrad = decltype(grad_c)::value;
    const u32x4 *ybase = stage ? ystage1 : ystage0;
    const float *cst = cstage[stage];
#pragma unroll
    for (int sb = 0; sb < C::kSub; ++sb) {
      const int tb = tile * C::kBT + sb * 32;
      if (tb >= p.nq) continue;  // the whole block is past N_Q: no e values, no dQ rows
      // 1. scores of the wave's 32 keys against the block's 32 queries,
      //    starting from the queries' row constants; inadmissible pairs
      //    (causal frontier, rows past N_Q, keys past N_K) start at -1e30.
      f32x16 s1, s2;
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
      const bool straddles =
          B.keys_past_end || tb + 31 > p.nq - 1 || (CAUSAL && tb < max(B.w0 + 31 - off, 0));
      if (straddles) {
        const int rel = tb + 4 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = rel + c_row(r, 0);
          const bool ok = B.srow < p.nk && t >= B.lim && t < p.nq;
          s1[r] = ok ? s1[r] : -1e30f;
          s2[r] = ok ? s2[r] : -1e30f;
        }
      }
      {
        const int arow = sb * 32 + col;
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          const int pos = arow * G::kChunks + swz<G::kChunks>(arow, frag_chunk<true, D>(h, cc));
          mfma_chunk<true>(*SK_L(&ybase[pos], 16, lds, kDyn, 3), xf1[cc], s1);
          mfma_chunk<true>(*SK_L(&ybase[C::kTileChunks + pos], 16, lds, kDyn, 3), xf2[cc], s2);
        }
      }
      // 2. e1, e2 packed to bf16: pk[ks][w] holds rows c_row(8ks + 2w, h)
      //    and c_row(8ks + 2w + 1, h).
      u32x4 pk1[2], pk2[2];
      {
        float e1[16], e2[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r0 = sb * 32 + g4 * 8 + 4 * h;
          const f32x4 KCv = *reinterpret_cast<const f32x4 *>(cst + 3 * C::kBT + r0);
          f32x4 Gv;
          if (GSIGN) Gv = *reinterpret_cast<const f32x4 *>(cst + 2 * C::kBT + r0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 4 * g4 + q;
            const float p1 = fast_exp2(s1[r] * c);
            const float p2 = kG2 ? fast_exp2(fmaf(s2[r], c, KCv[q])) : 0.f;
            if (GSIGN) {
              const float gp1 = p1 * Gv[q];
              e2[r] = fmaf(p2, Gv[q], -gp1);
              e1[r] = gp1 * (s1[r] - s2[r]);
            } else {
              e2[r] = p2 - p1;
              e1[r] = p1 * (s1[r] - s2[r]);
            }
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pk1[ks][w] = pack_bf16(e1[8 * ks + 2 * w], e1[8 * ks + 2 * w + 1]);
            pk2[ks][w] = pack_bf16(e2[8 * ks + 2 * w], e2[8 * ks + 2 * w + 1]);
          }
      }
      // 3. dK_t^T += Q_t^T e_t: Q_t^T from transposing reads of the tile
      //    (lane (s, grp) supplies query row sb*32 + 16ks + 8t + 4h + s/4,
      //    columns m*32 + 16(grp&1) + 4(s&3) .. +3).
      auto grad = [&](const char *yb, const u32x4 (&pk)[2], f32x16 (&acc)[kMB]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int m = 0; m < kMB; ++m) {
            const int d0 = m * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
            u32x4 a;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int row = sb * 32 + 16 * ks + 8 * t + 4 * h + (s16 >> 2);
              const u32x2 v = read_tr(SK_L((yb + (row * G::kChunks + swz<G::kChunks>(row, d0 >> 3)) * 16 + (d0 & 7) * 2), 8, lds, kDyn, 3));
              a[2 * t] = v[0];
              a[2 * t + 1] = v[1];
            }
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, pk[ks]), acc[m], 0, 0, 0);
          }
      };
      if constexpr (kInlineGrad) {
        if (kG1) grad(reinterpret_cast<const char *>(ybase), pk1, acc1);
        if (kG2) grad(reinterpret_cast<const char *>(ybase + C::kTileChunks), pk2, acc2);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          pks[sb][0][ks] = pk1[ks];
          pks[sb][1][ks] = pk2[ks];
        }
      }
      // 4. e_t -> the e buffer, row = the lane's key (within the workgroup),
      //    4 consecutive queries (32 sb + 8 g4 + 4 h ..) per store.
      {
        const int key = wave * 32 + col;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q = sb * 32 + 8 * g4 + 4 * h;
          const int ks = g4 >> 1, w = 2 * (g4 & 1);
          if (kG1)
            *reinterpret_cast<u32x2 *>(SK_L(ebuf + ebyte(key, q), 8, lds, kDyn, 3)) = u32x2{pk1[ks][w], pk1[ks][w + 1]};
          if (kG2)
            *reinterpret_cast<u32x2 *>(SK_L(ebuf + C::kEBytes + ebyte(key, q), 8, lds, kDyn, 3)) =
                u32x2{pk2[ks][w], pk2[ks][w + 1]};
        }
      }
    }
  };

  // 5. dQ_t block (32 queries x the wave's 32 columns of d) = e_t x K_t over
  //    the wave's key group, added to `a`.  A operand: e_t with lane =
  //    query, 8 keys per half, by transposing reads of the [key][query]
  //    buffer (lane (s, grp) supplies key row 16ks + 8t + 4h + s/4, queries
  //    32sb + 16(grp&1) + 4(s&3) .. +3).
  auto dq_product = [&](int sb, const char *eb, const u32x4 (&kt)[C::kKSteps], f32x16 a) {
    const int qa = sb * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
      u32x4 e;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = kg * C::kGroupKeys + 16 * ks + 8 * t + 4 * h + (s16 >> 2);
        const u32x2 v = read_tr(SK_L(eb + ebyte(key, qa), 8, lds, kDyn, 3));
        e[2 * t] = v[0];
        e[2 * t + 1] = v[1];
      }
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, e), __builtin_bit_cast(bf16x8, kt[ks]),
                                                  a, 0, 0, 0);
    }
    return a;
  };
  // The fp32 sums += a, with atomics.  a[r]: query tile*64 + 32 sb +
  // c_row(r, h), column mb*32 + col.  The row offset is made opaque to the
  // compiler, so that the 16 addresses are formed here rather than kept
  // live (as 32 registers) across the one-tile form's loop over key blocks.
  auto dq_atomics = [&](int tile, int sb, const f32x16 &a, float *ws) {
    const int qb = tile * C::kBT + sb * 32;
    size_t rowoff = (size_t(bh) * p.nq + qb) * D + mb * 32 + col;
    asm volatile("" : "+v"(rowoff));
    float *base = ws + rowoff;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = c_row(r, h);
      if (qb + q < p.nq && SK_OK(base + size_t(q) * D, 4, ws, p.xw, 3)) unsafeAtomicAdd(base + size_t(q) * D, a[r]);
    }
  };
  auto tile_dq = [&](int tile) {
#pragma unroll
    for (int sb = 0; sb < C::kSub; ++sb) {
      if (tile * C::kBT + sb * 32 >= p.nq) continue;  // skipped in tile_work as well
      if (kG1) dq_atomics(tile, sb, dq_product(sb, ebuf, kt1, f32x16{}), p.ws1);
      if (kG2) dq_atomics(tile, sb, dq_product(sb, ebuf + C::kEBytes, kt2, f32x16{}), p.ws2);
    }
  };

  // dK write-out of block B: dK1 = scale^2 acc1, dK2 = scale acc2 (g is
  // inside e).
  auto store_dk = [&](const Blk &B) {
    if (B.srow >= p.nk) return;
    const size_t ro = koff + size_t(B.srow) * G::kRowBytes;
    auto store = [&](char *O, float f, const f32x16 (&A)[kMB]) {
#pragma unroll
      for (int m = 0; m < kMB; ++m)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = m * 32 + g4 * 8 + 4 * h;
          if (SK_OK(O + ro + d0 * 2, 8, O, p.xk, 3))
            *reinterpret_cast<u32x2 *>(O + ro + d0 * 2) =
              u32x2{pack_bf16(A[m][4 * g4] * f, A[m][4 * g4 + 1] * f), pack_bf16(A[m][4 * g4 + 2] * f, A[m][4 * g4 + 3] * f)};
        }
    };
    if (kG1) store(p.dk1, p.scale * p.scale, acc1);
    if (kG2) store(p.dk2, p.scale, acc2);
  };
  // The one-tile form's dK of block B (query tile in stage 0): dK_t^T =
  // Q_t^T e_t from the packed e values, one tensor and two 32-column slices
  // of d at a time, each pair written out as soon as it is complete: 32
  // accumulator registers instead of 128, and every store burst covers whole
  // 128-byte lines of the key rows (64-byte halves written apart measured
  // 0.35 GB of extra HBM writes at 64 queries x 64K keys x 32 heads).  Each
  // slice's products run in the order step 3 takes them, so the results are
  // the same bits.
  auto dk_by_slices = [&](const Blk &B, const PackedE &pks) {
    const size_t ro = koff + size_t(min(B.srow, p.nk - 1)) * G::kRowBytes;
    auto tensor = [&](int t, const char *yb, char *O, float f) {
#pragma unroll
      for (int mp = 0; mp < kMB; mp += 2) {
        f32x16 a[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int sb = 0; sb < C::kSub; ++sb) {
          if (sb * 32 >= p.nq) continue;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int d0 = (mp + j) * 32 + 16 * (grp & 1) + 4 * (s16 & 3);
              u32x4 fq;
#pragma unroll
              for (int tt = 0; tt < 2; ++tt) {
                const int row = sb * 32 + 16 * ks + 8 * tt + 4 * h + (s16 >> 2);
                const u32x2 v = read_tr(SK_L((yb + (row * G::kChunks + swz<G::kChunks>(row, d0 >> 3)) * 16 + (d0 & 7) * 2), 8, lds, kDyn, 3));
                fq[2 * tt] = v[0];
                fq[2 * tt + 1] = v[1];
              }
              a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fq),
                                                             __builtin_bit_cast(bf16x8, pks[sb][t][ks]), a[j], 0, 0, 0);
            }
        }
        if (B.srow < p.nk) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int dc = (mp + j) * 32 + g4 * 8 + 4 * h;
              if (SK_OK(O + ro + dc * 2, 8, O, p.xk, 3))
                *reinterpret_cast<u32x2 *>(O + ro + dc * 2) =
                  u32x2{pack_bf16(a[j][4 * g4] * f, a[j][4 * g4 + 1] * f), pack_bf16(a[j][4 * g4 + 2] * f, a[j][4 * g4 + 3] * f)};
            }
        }
      }
    };
    if (kG1) tensor(0, reinterpret_cast<const char *>(ystage0), p.dk1, p.scale * p.scale);
    if (kG2) tensor(1, reinterpret_cast<const char *>(ystage0 + C::kTileChunks), p.dk2, p.scale);
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      acc1[m] = f32x16{};
      acc2[m] = f32x16{};
    }
  };

  if constexpr (MULTI) {
    // One query tile (N_Q <= kBT: every key block's causal frontier lies in
    // it), loaded once; the key blocks follow one another, each block's
    // stationary tiles copied while the previous block is worked on.
    // The copies of block kb + 1 are waited for at the end of block kb, so
    // that they overlap all of its products; the wait also covers block kb's
    // dK stores (one counter for loads and stores), which then overlap its
    // dQ products (1-2% faster at 1-64 queries x 64K keys than waiting after
    // the scores, where the stores had a whole block).  The dQ blocks are summed over the workgroup's key
    // blocks in registers and added to the fp32 sums once, at the end: the
    // atomics fall kbpw-fold.
    if (blk0 >= blk1) return;
    load_x(blk0, std::false_type{});
    issue(0, 0);
    cwrite(0, 0);
    __syncthreads();  // the first stationary tiles, the query tile and its constants
    f32x16 dqa1[C::kSub], dqa2[C::kSub];
#pragma unroll
    for (int sb = 0; sb < C::kSub; ++sb) dqa1[sb] = dqa2[sb] = f32x16{};
    for (int kb = blk0; kb < blk1; ++kb) {
      const Blk B = blk_state(kb);
      read_frags();
      __syncthreads();  // every wave has its fragments: the stationary space is free
      if (kb + 1 < blk1) load_x(kb + 1, std::true_type{});
      PackedE pks;
      tile_work(0, 0, B, std::false_type{}, pks);
      __syncthreads();  // every wave's e blocks are in the buffer
      dk_by_slices(B, pks);
#pragma unroll
      for (int sb = 0; sb < C::kSub; ++sb) {
        if (sb * 32 >= p.nq) continue;
        if (kG1) dqa1[sb] = dq_product(sb, ebuf, kt1, dqa1[sb]);
        if (kG2) dqa2[sb] = dq_product(sb, ebuf + C::kEBytes, kt2, dqa2[sb]);
      }
      vmcnt0_wait();    // block kb + 1's stationary tiles have landed
      __syncthreads();  // the e buffer is free again; those tiles are published
    }
#pragma unroll
    for (int sb = 0; sb < C::kSub; ++sb) {
      if (sb * 32 >= p.nq) continue;
      if (kG1) dq_atomics(0, sb, dqa1[sb], p.ws1);
      if (kG2) dq_atomics(0, sb, dqa2[sb], p.ws2);
    }
    return;
  }

  const Blk B = blk_state(blk0);
  // Streamed query range: from the workgroup's causal frontier to N_Q.
  const int t_begin = CAUSAL ? max(0, B.s0 - off) : 0;
  const int tile0 = t_begin / C::kBT;
  const int tile1 = (p.nq + C::kBT - 1) / C::kBT;
  const int ntiles = max(tile1 - tile0, 0);

  load_x(blk0, std::false_type{});
  if (ntiles > 0) {
    issue(tile0, 0);
    cwrite(tile0, 0);
  }
  __syncthreads();  // the stationary tiles, the first query tile and its constants
  read_frags();
  __syncthreads();  // everyone has its fragments: the space is free for stage 1 and the e buffers
  zero_acc();

  for (int it = 0; it < ntiles; ++it) {
    const int tile = tile0 + it;
    const int stage = it & 1;
    if (it + 1 < ntiles) issue(tile + 1, stage ^ 1);
    PackedE unused;
    tile_work(tile, stage, B, std::true_type{}, unused);
    __syncthreads();  // every wave's e blocks of this tile are in the buffer
    tile_dq(tile);
    if (it + 1 < ntiles) cwrite(tile + 1, stage ^ 1);
    __syncthreads();  // the next tile's copies and constants; the e buffer is free again
  }
  store_dk(B);
}

// Zeroes n4 float4 values.
__global__ __launch_bounds__(256) void zero_kernel(f32x4 *x, size_t n4 SK_DBG_ARGS(size_t xw)) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += size_t(gridDim.x) * 256)
    if (SK_OK(x + i, 16, x, xw, 3)) x[i] = f32x4{};
}

// dq = f * ws, fp32 -> bf16 (nearest even); 4 values per thread.  blockIdx.y
// picks the gradient, so both requested gradients take one launch.
__global__ __launch_bounds__(256) void convert_kernel(const f32x4 *ws0, float f0, u32x2 *out0, const f32x4 *ws1,
                                                      float f1, u32x2 *out1, size_t n4 SK_DBG_ARGS(size_t xw, size_t xo)) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 *ws = blockIdx.y ? ws1 : ws0;
  const float f = blockIdx.y ? f1 : f0;
  u32x2 *out = blockIdx.y ? out1 : out0;
  const f32x4 v = *SK_G(&ws[i], 16, ws, xw, 3);
  if (SK_OK(out + i, 8, out, xo, 3)) out[i] = u32x2{pack_bf16(v[0] * f, v[1] * f), pack_bf16(v[2] * f, v[3] * f)};
}

template <int D, bool CAUSAL, int MASK, bool GSIGN>
hipError_t launch_fused_t(const BwdArgs &a, float *ws, hipStream_t stream) {
  using C = FusedCfg<D>;
  FusedParams p;
  p.q1 = static_cast<const char *>(a.q1);
  p.k1 = static_cast<const char *>(a.k1);
  p.q2 = static_cast<const char *>(a.q2);
  p.k2 = static_cast<const char *>(a.k2);
  p.kl = a.kl;
  p.lse1 = a.lse1;
  p.lse2 = a.lse2;
  p.dkl = a.dkl;
  p.dk1 = static_cast<char *>(a.dk1);
  p.dk2 = static_cast<char *>(a.dk2);
  const size_t n = size_t(a.bh) * a.nq * D;  // values per requested gradient
  p.ws1 = ws;
  p.ws2 = ws + ((MASK & 1) ? n : 0);
  p.nq = a.nq;
  p.nk = a.nk;
  p.nsb = (a.nk + C::kBS - 1) / C::kBS;
  // With one query tile, a workgroup walks up to 64 key blocks, as many as
  // leave one round of workgroups (one per CU): fewer prologues and rounds of
  // atomics than two rounds of at most 16 blocks (3-11% faster from 4 heads x
  // 64K keys to 32 heads x 256K keys; with no cap, 5% slower at one query x
  // 32 heads x 256K keys).  More tiles, or none (dK is then written as
  // zeros): one block.
  const bool multi = a.nq >= 1 && a.nq <= C::kBT;
  const long long nblk = (long long)p.nsb * a.bh;
  p.kbpw = multi ? int(std::max(1LL, std::min(64LL, nblk / 256))) : 1;
  const int ngrp = (p.nsb + p.kbpw - 1) / p.kbpw;
  p.scale = a.scale;
  p.c = float(double(a.scale) * 1.4426950408889634);
  p.inv_scale = float(1.0 / double(a.scale));
#ifdef STREAMKL_DEBUG
  p.xq = size_t(a.bh) * a.nq * C::G::kRowBytes;
  p.xk = size_t(a.bh) * a.nk * C::G::kRowBytes;
  p.xr = size_t(a.bh) * a.nq * sizeof(float);
  p.xw = n * sizeof(float);
#endif
  const int ngrad = ((MASK & 1) ? 1 : 0) + ((MASK & 2) ? 1 : 0);
  const size_t n4 = n / 4;  // D is a multiple of 4
  if (n4 > 0) {
    const size_t zb = std::min<size_t>((n4 * ngrad + 255) / 256, 4096);
    zero_kernel<<<dim3(unsigned(zb)), dim3(256), 0, stream>>>(reinterpret_cast<f32x4 *>(ws),
                                                            n4 * ngrad SK_DBG_ARGS(n * ngrad * sizeof(float)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long blocks = (long long)ngrp * a.bh;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  if (blocks > 0) {
    const void *fn = multi ? reinterpret_cast<const void *>(&fused_bwd_kernel<D, CAUSAL, MASK, GSIGN, true>)
                           : reinterpret_cast<const void *>(&fused_bwd_kernel<D, CAUSAL, MASK, GSIGN, false>);
    const int lds_bytes = multi ? C::kLdsBytesM : C::kLdsBytes;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    void *args[] = {&p};
    e = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(C::kThreads), args, lds_bytes, stream);
    if (e != hipSuccess) return e;
  }
  if (n4 > 0) {
    const size_t cb = (n4 + 255) / 256;
    if (cb > size_t(INT_MAX)) return hipErrorInvalidConfiguration;
    // Gradient 0 of the launch is dq1 when requested, else dq2.
    const f32x4 *w0 = reinterpret_cast<const f32x4 *>((MASK & 1) ? p.ws1 : p.ws2);
    const float f0 = (MASK & 1) ? a.scale * a.scale : a.scale;
    u32x2 *o0 = static_cast<u32x2 *>((MASK & 1) ? a.dq1 : a.dq2);
    convert_kernel<<<dim3(unsigned(cb), unsigned(ngrad)), dim3(256), 0, stream>>>(
        w0, f0, o0, reinterpret_cast<const f32x4 *>(p.ws2), a.scale, static_cast<u32x2 *>(a.dq2),
        n4 SK_DBG_ARGS(n * sizeof(float), p.xq));
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fused_masks(const BwdArgs &a, float *ws, hipStream_t s) {
  const bool gsign = a.dkl != nullptr;
  switch (a.grad_mask) {
    case 1: return gsign ? launch_fused_t<D, CAUSAL, 1, true>(a, ws, s) : launch_fused_t<D, CAUSAL, 1, false>(a, ws, s);
    case 2: return gsign ? launch_fused_t<D, CAUSAL, 2, true>(a, ws, s) : launch_fused_t<D, CAUSAL, 2, false>(a, ws, s);
    default: return gsign ? launch_fused_t<D, CAUSAL, 3, true>(a, ws, s) : launch_fused_t<D, CAUSAL, 3, false>(a, ws, s);
  }
}

}  // namespace

size_t bwd_fused_workspace_floats(int bh, int nq, int d, int grad_mask) {
  if (bh <= 0 || nq <= 0) return 0;
  const int ngrad = ((grad_mask & 1) ? 1 : 0) + ((grad_mask & 2) ? 1 : 0);
  return size_t(bh) * size_t(nq) * size_t(d) * size_t(ngrad);
}

hipError_t launch_bwd_fused(const BwdArgs &a, float *ws, hipStream_t stream) {
  if (!a.bf16) return hipErrorInvalidValue;
  if (a.d == 64) return a.causal ? launch_fused_masks<64, true>(a, ws, stream) : launch_fused_masks<64, false>(a, ws, stream);
  return a.causal ? launch_fused_masks<128, true>(a, ws, stream) : launch_fused_masks<128, false>(a, ws, stream);
}

#ifdef STREAMKL_DEBUG
unsigned dbg_take_bwd_fused() { return dbg_take(); }
#endif
}  // namespace streamkl
