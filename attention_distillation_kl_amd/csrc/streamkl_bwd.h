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
//   ROLE_DQ: a workgroup owns 128 query rows ("stationary") and streams key
//            tiles ("streamed") up to its causal frontier; it accumulates dQ.
//   ROLE_DK: a workgroup owns 128 key rows and streams query tiles from its
//            causal frontier to N_Q; it accumulates dK.
// Both recompute S1, S2; neither needs atomics or workspace, and results are
// bitwise deterministic.
//
// Per 32-row streamed tile each wave:
//   1. S_t^T block (32 streamed x 32 stationary) = Y_t X_t^T with the
//      stationary fragments X_t held in registers (B operand) and the
//      streamed rows Y_t read from LDS (A operand): each lane owns one
//      stationary row and 16 streamed rows of the block;
//   2. P_t = exp2(s_t * scale*log2e - LSE_t*log2e + log2|g|), dS_t in fp32;
//   3. dX_t^T (d x 32 stationary) += Y_t^T dS_t, with Y_t^T read from a
//      transposed LDS copy whose row order matches the register order of dS
//      (so dS feeds the product as the B operand with no shuffles).
// The sign of g is applied to dQ at the end (ROLE_DQ) or folded into the
// transposed query copy (ROLE_DK); |g| is folded into the exponent.
#pragma once

#include "streamkl_device.h"
#include "streamkl_launch.h"

#include <climits>
#include <cmath>

namespace streamkl {

enum { ROLE_DQ = 0, ROLE_DK = 1 };

template <bool BF16, int D>
struct BwdCfg {
  using G = RowGeom<BF16, D>;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBS = 32 * kWaves;   // stationary rows per workgroup
  static constexpr int kBT = 32;            // streamed rows per LDS tile
  static constexpr int kRowChunks = kBT * G::kChunks;             // row-major copy, per tensor
  static constexpr int kTCPR = kBT * G::kElemBytes / 16;          // chunks per transposed row
  static constexpr int kTChunks = D * kTCPR;                      // transposed copy, per tensor
  static constexpr int kCstChunks = 3 * kBT / 4;                  // 3 fp32 arrays of kBT
  // stage layout in 16-B chunks: [Y1][Y2][Y1^T][Y2^T][L1'|L2'|delta]
  static constexpr int kOffY2 = kRowChunks;
  static constexpr int kOffT1 = 2 * kRowChunks;
  static constexpr int kOffT2 = 2 * kRowChunks + kTChunks;
  static constexpr int kOffCst = 2 * kRowChunks + 2 * kTChunks;
  static constexpr int kStage = kOffCst + kCstChunks;
  static constexpr size_t kLdsBytes = size_t(2) * kStage * 16;
  // staging unit: 4 consecutive streamed rows x one 16-B chunk of one tensor
  static constexpr int kBlocksPerTensor = (kBT / 4) * G::kChunks;
  static constexpr int kBlocks = 2 * kBlocksPerTensor;
  static constexpr int kBlocksPerThread = (kBlocks + kThreads - 1) / kThreads;
};

struct BwdParams {
  const char *q1, *k1, *q2, *k2;
  const float *kl, *lse1, *lse2, *dkl;
  char *dq1, *dk1, *dq2, *dk2;
  int nq, nk, nsb;  // nsb: stationary blocks per head
  float scale, c;   // c = scale * log2(e)
};

// Per-row constants of the recompute: P_t |g| = exp2(s_t c - Lt'),
// Lt' = LSE_t log2(e) - log2|g|, and delta = KL + LSE1 - LSE2.
__device__ __forceinline__ void row_constants(const BwdParams &p, size_t i, float &L1, float &L2,
                                              float &delta, float &sgn) {
  const float lse1 = p.lse1[i], lse2 = p.lse2[i], kl = p.kl[i];
  float lg = 0.f;
  sgn = 1.f;
  if (p.dkl) {
    const float g = p.dkl[i];
    lg = log2f(fabsf(g));  // g == 0 -> -inf -> P|g| = 0
    sgn = g < 0.f ? -1.f : 1.f;
  }
  L1 = lse1 * kLog2e - lg;
  L2 = lse2 * kLog2e - lg;
  delta = kl + lse1 - lse2;
}

template <bool BF16, int D, bool CAUSAL, int ROLE, int MASK>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_kernel(BwdParams p) {
  using C = BwdCfg<BF16, D>;
  using G = typename C::G;
  constexpr bool kG1 = (MASK & 1) != 0;
  constexpr bool kG2 = (MASK & 2) != 0;
  constexpr int kMB = D / 32;  // 32-row blocks of d in the gradient accumulators
  extern __shared__ u32x4 lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = bid / p.nsb;
  const int sbr = bid - bh * p.nsb;
  // Longest rows first: for causal problems the last query blocks (ROLE_DQ)
  // and the first key blocks (ROLE_DK) see the most partners.
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
  const int w0 = s0 + wave * 32;
  const int srow = w0 + col;
  const bool wave_active = w0 < ns;

  u32x4 xf1[G::kLaneChunks], xf2[G::kLaneChunks];
  if (srow < ns) {
    const u32x4 *r1 = reinterpret_cast<const u32x4 *>(X1 + xoff + size_t(srow) * G::kRowBytes);
    const u32x4 *r2 = reinterpret_cast<const u32x4 *>(X2 + xoff + size_t(srow) * G::kRowBytes);
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) {
      xf1[c] = r1[frag_chunk<BF16, D>(h, c)];
      xf2[c] = r2[frag_chunk<BF16, D>(h, c)];
    }
  } else {
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) xf1[c] = xf2[c] = zero4();
  }

  // ROLE_DQ: the lane's query is stationary, its constants live in registers.
  float rl1 = INFINITY, rl2 = INFINITY, rdelta = 0.f, rsign = 1.f;
  if (ROLE == ROLE_DQ && srow < p.nq) row_constants(p, size_t(bh) * p.nq + srow, rl1, rl2, rdelta, rsign);

  // Streamed range and per-element admissibility.
  //   ROLE_DQ (streamed keys tau, stationary query sigma): tau <= sigma + off, tau < N_K.
  //   ROLE_DK (streamed queries tau, stationary key sigma): tau >= sigma - off, tau < N_Q.
  int t_begin = 0, t_end = nt;
  if (CAUSAL) {
    if (ROLE == ROLE_DQ) t_end = min(p.nk, min(s0 + C::kBS, p.nq) + off);
    else t_begin = max(0, s0 - off);
  }
  const int tile0 = t_begin / C::kBT;
  const int tile1 = (t_end + C::kBT - 1) / C::kBT;
  int lim;       // ROLE_DQ: last admissible key; ROLE_DK: first admissible query
  int w_easy;    // wave-uniform bound beyond which no element needs a mask
  int w_any;     // wave-uniform bound beyond which the whole tile is masked
  if (ROLE == ROLE_DQ) {
    lim = CAUSAL ? min(srow + off, p.nk - 1) : p.nk - 1;
    w_easy = CAUSAL ? min(w0 + off, p.nk - 1) : p.nk - 1;
    w_any = CAUSAL ? min(w0 + 31 + off, p.nk - 1) : p.nk - 1;
  } else {
    lim = CAUSAL ? max(srow - off, 0) : 0;
    w_easy = CAUSAL ? max(w0 + 31 - off, 0) : 0;
    w_any = CAUSAL ? max(w0 - off, 0) : 0;
  }

  // ---------------------------------------------------------------- staging
  u32x4 st[C::kBlocksPerThread][4];
  uint32_t sgnmask[C::kBlocksPerThread][2];  // ROLE_DK: sign of g folded into Y^T

  auto gload = [&](int tile) {
    const int tb = tile * C::kBT;
#pragma unroll
    for (int bi = 0; bi < C::kBlocksPerThread; ++bi) {
      const int blk = tid + bi * C::kThreads;
      if (blk < C::kBlocks) {
        const int t = blk / C::kBlocksPerTensor;
        const int rem = blk - t * C::kBlocksPerTensor;
        const int rg = rem / G::kChunks, ch = rem - rg * G::kChunks;
        const char *Y = t ? Y2 : Y1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = tb + 4 * rg + e;
          st[bi][e] = row < nt ? *reinterpret_cast<const u32x4 *>(Y + size_t(row) * G::kRowBytes + ch * 16)
                               : zero4();
        }
        sgnmask[bi][0] = sgnmask[bi][1] = 0u;
        if (ROLE == ROLE_DK && p.dkl) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = tb + 4 * rg + e;
            const bool neg = row < p.nq && p.dkl[size_t(bh) * p.nq + row] < 0.f;
            if (BF16) sgnmask[bi][e >> 1] |= neg ? (0x8000u << (16 * (e & 1))) : 0u;
            else sgnmask[bi][0] |= neg ? (1u << e) : 0u;
          }
        }
      }
    }
  };

  float cst_l1 = INFINITY, cst_l2 = INFINITY, cst_d = 0.f;  // ROLE_DK row constants in flight
  auto cload = [&](int tile) {
    if (ROLE == ROLE_DK && tid < C::kBT) {
      const int row = tile * C::kBT + tid;
      float sg;
      cst_l1 = INFINITY;
      cst_l2 = INFINITY;
      cst_d = 0.f;
      if (row < p.nq) row_constants(p, size_t(bh) * p.nq + row, cst_l1, cst_l2, cst_d, sg);
    }
  };

  auto swrite = [&](int stage) {
    u32x4 *base = lds + stage * C::kStage;
#pragma unroll
    for (int bi = 0; bi < C::kBlocksPerThread; ++bi) {
      const int blk = tid + bi * C::kThreads;
      if (blk < C::kBlocks) {
        const int t = blk / C::kBlocksPerTensor;
        const int rem = blk - t * C::kBlocksPerTensor;
        const int rg = rem / G::kChunks, ch = rem - rg * G::kChunks;
        u32x4 *ym = base + (t ? C::kOffY2 : 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * rg + e;
          ym[row * G::kChunks + swz<G::kChunks>(row, ch)] = st[bi][e];
        }
        const bool want_t = t ? kG2 : kG1;
        if (want_t) {
          u32x4 *yt = base + (t ? C::kOffT2 : C::kOffT1);
          // rows 4rg..4rg+3 sit at 4 consecutive positions of the transposed layout
          const int pos0 = 16 * ((4 * rg) >> 4) + tpos((4 * rg) & 15);
          if constexpr (BF16) {
            // element e of the chunk is d = 8 ch + e; pack (row0,row1), (row2,row3)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int w = e >> 1;
              const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
              uint32_t lo = __builtin_amdgcn_perm(st[bi][1][w], st[bi][0][w], sel);
              uint32_t hi = __builtin_amdgcn_perm(st[bi][3][w], st[bi][2][w], sel);
              lo ^= sgnmask[bi][0];
              hi ^= sgnmask[bi][1];
              const int drow = 8 * ch + e;
              const int byte = pos0 * 2;  // 8-B aligned inside a 16-B chunk
              const int pch = swz<C::kTCPR>(drow, byte >> 4);
              uint32_t *dst = reinterpret_cast<uint32_t *>(yt + drow * C::kTCPR + pch) + ((byte & 15) >> 2);
              *reinterpret_cast<u32x2 *>(dst) = u32x2{lo, hi};
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              u32x4 v{st[bi][0][e], st[bi][1][e], st[bi][2][e], st[bi][3][e]};
#pragma unroll
              for (int q = 0; q < 4; ++q) v[q] ^= ((sgnmask[bi][0] >> q) & 1u) << 31;
              const int drow = 4 * ch + e;
              const int pch = swz<C::kTCPR>(drow, pos0 >> 2);
              yt[drow * C::kTCPR + pch] = v;
            }
          }
        }
      }
    }
    if (ROLE == ROLE_DK && tid < C::kBT) {
      float *cst = reinterpret_cast<float *>(base + C::kOffCst);
      cst[tid] = cst_l1;
      cst[C::kBT + tid] = cst_l2;
      cst[2 * C::kBT + tid] = cst_d;
    }
  };

  f32x16 acc1[kMB], acc2[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    acc1[mb] = f32x16{};
    acc2[mb] = f32x16{};
  }

  const float c = p.c, scale = p.scale;
  const int ntiles = tile1 - tile0;
  if (ntiles > 0) {
    gload(tile0);
    cload(tile0);
    swrite(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int tile = tile0 + it;
    const int stage = it & 1;
    if (it + 1 < ntiles) {
      gload(tile + 1);
      cload(tile + 1);
    }
    const int tb = tile * C::kBT;
    const bool tile_live = ROLE == ROLE_DQ ? tb <= w_any : tb + C::kBT - 1 >= w_any;

    if (wave_active && tile_live) {
      const u32x4 *base = lds + stage * C::kStage;
      // 1. recompute the two score blocks
      f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
      for (int cc = 0; cc < G::kLaneChunks; ++cc) {
        const int pos = col * G::kChunks + swz<G::kChunks>(col, frag_chunk<BF16, D>(h, cc));
        mfma_chunk<BF16>(base[pos], xf1[cc], s1);
        mfma_chunk<BF16>(base[C::kOffY2 + pos], xf2[cc], s2);
      }

      // 2. regenerate P and form dS (fp32)
      bool need_mask;
      if (ROLE == ROLE_DQ) need_mask = tb + C::kBT - 1 > w_easy;
      else need_mask = (CAUSAL && tb < w_easy) || tb + C::kBT > p.nq;
      float ds1[16], ds2[16];
      const float *cst = reinterpret_cast<const float *>(base + C::kOffCst);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 L1v, L2v, Dv;
        if (ROLE == ROLE_DK) {
          const int r0 = g4 * 8 + 4 * h;
          L1v = *reinterpret_cast<const f32x4 *>(cst + r0);
          L2v = *reinterpret_cast<const f32x4 *>(cst + C::kBT + r0);
          Dv = *reinterpret_cast<const f32x4 *>(cst + 2 * C::kBT + r0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = g4 * 4 + q;
          const float L1 = ROLE == ROLE_DK ? L1v[q] : rl1;
          const float L2 = ROLE == ROLE_DK ? L2v[q] : rl2;
          const float dl = ROLE == ROLE_DK ? Dv[q] : rdelta;
          float p1 = fast_exp2(fmaf(s1[r], c, -L1));
          float p2 = kG2 ? fast_exp2(fmaf(s2[r], c, -L2)) : 0.f;
          if (need_mask) {
            const int tau = tb + c_row(r, h);
            const bool ok = ROLE == ROLE_DQ ? tau <= lim : (tau >= lim && tau < p.nq);
            p1 = ok ? p1 : 0.f;
            p2 = ok ? p2 : 0.f;
          }
          ds2[r] = p2 - p1;
          ds1[r] = p1 * fmaf(s1[r] - s2[r], scale, -dl);
        }
      }

      // 3. gradient products: dX_t^T += Y_t^T dS_t
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (BF16) {
          u32x4 b1, b2;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            b1[w] = pack_bf16(ds1[8 * ks + 2 * w], ds1[8 * ks + 2 * w + 1]);
            b2[w] = pack_bf16(ds2[8 * ks + 2 * w], ds2[8 * ks + 2 * w + 1]);
          }
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            const int drow = mb * 32 + col;
            const int pch = swz<C::kTCPR>(drow, 2 * ks + h);
            if (kG1) {
              const u32x4 a = base[C::kOffT1 + drow * C::kTCPR + pch];
              acc1[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b1), acc1[mb], 0, 0, 0);
            }
            if (kG2) {
              const u32x4 a = base[C::kOffT2 + drow * C::kTCPR + pch];
              acc2[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b2), acc2[mb], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            const int drow = mb * 32 + col;
            const int pc0 = swz<C::kTCPR>(drow, 4 * ks + 2 * h);
            const int pc1 = swz<C::kTCPR>(drow, 4 * ks + 2 * h + 1);
            if (kG1) {
              const u32x4 a0 = base[C::kOffT1 + drow * C::kTCPR + pc0];
              const u32x4 a1 = base[C::kOffT1 + drow * C::kTCPR + pc1];
#pragma unroll
              for (int j = 0; j < 8; ++j)
                acc1[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    u2f(j < 4 ? a0[j] : a1[j - 4]), ds1[8 * ks + j], acc1[mb], 0, 0, 0);
            }
            if (kG2) {
              const u32x4 a0 = base[C::kOffT2 + drow * C::kTCPR + pc0];
              const u32x4 a1 = base[C::kOffT2 + drow * C::kTCPR + pc1];
#pragma unroll
              for (int j = 0; j < 8; ++j)
                acc2[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    u2f(j < 4 ? a0[j] : a1[j - 4]), ds2[8 * ks + j], acc2[mb], 0, 0, 0);
            }
          }
        }
      }
    }

    if (it + 1 < ntiles) swrite(stage ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- write-out
  if (srow < ns) {
    const float f = scale * (ROLE == ROLE_DQ ? rsign : 1.f);
    char *O1 = ROLE == ROLE_DQ ? p.dq1 : p.dk1;
    char *O2 = ROLE == ROLE_DQ ? p.dq2 : p.dk2;
    const size_t ro = (size_t(bh) * ns + srow) * G::kRowBytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 0 && !kG1) continue;
      if (t == 1 && !kG2) continue;
      char *O = (t ? O2 : O1) + ro;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = mb * 32 + g4 * 8 + 4 * h;
          const f32x16 &A = t ? acc2[mb] : acc1[mb];
          const float v0 = A[4 * g4] * f, v1 = A[4 * g4 + 1] * f;
          const float v2 = A[4 * g4 + 2] * f, v3 = A[4 * g4 + 3] * f;
          if constexpr (BF16) {
            *reinterpret_cast<u32x2 *>(O + d0 * 2) = u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
          } else {
            *reinterpret_cast<f32x4 *>(O + d0 * 4) = f32x4{v0, v1, v2, v3};
          }
        }
    }
  }
}

template <bool BF16, int D, bool CAUSAL, int ROLE, int MASK>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream) {
  using C = BwdCfg<BF16, D>;
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
  const long long blocks = (long long)p.nsb * a.bh;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const void *fn = reinterpret_cast<const void *>(&bwd_kernel<BF16, D, CAUSAL, ROLE, MASK>);
  if (C::kLdsBytes > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(C::kLdsBytes));
    if (e != hipSuccess) return e;
  }
  void *args[] = {&p};
  return hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(C::kThreads), args, C::kLdsBytes, stream);
}

template <int ROLE>
hipError_t launch_bwd_role(const BwdArgs &a, hipStream_t s) {
#define STREAMKL_BWD_MASKS(BF, DD, CA)                                  \
  switch (a.grad_mask) {                                                \
    case 1: return launch_bwd_t<BF, DD, CA, ROLE, 1>(a, s);             \
    case 2: return launch_bwd_t<BF, DD, CA, ROLE, 2>(a, s);             \
    default: return launch_bwd_t<BF, DD, CA, ROLE, 3>(a, s);            \
  }
  if (a.bf16) {
    if (a.d == 64) {
      if (a.causal) { STREAMKL_BWD_MASKS(true, 64, true) } else { STREAMKL_BWD_MASKS(true, 64, false) }
    } else {
      if (a.causal) { STREAMKL_BWD_MASKS(true, 128, true) } else { STREAMKL_BWD_MASKS(true, 128, false) }
    }
  } else {
    if (a.d == 64) {
      if (a.causal) { STREAMKL_BWD_MASKS(false, 64, true) } else { STREAMKL_BWD_MASKS(false, 64, false) }
    } else {
      if (a.causal) { STREAMKL_BWD_MASKS(false, 128, true) } else { STREAMKL_BWD_MASKS(false, 128, false) }
    }
  }
#undef STREAMKL_BWD_MASKS
}

}  // namespace streamkl
