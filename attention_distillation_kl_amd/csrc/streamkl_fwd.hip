// streamkl_fwd.hip -- fused single-pass attention-KL forward kernel (gfx950).
//
// StreamKL summary page (gist.science 2606.20005), "Formulazione Online":
// KL(P1 || P2) of one query row is rewritten in terms of five running row
// scalars -- the running maxima m1, m2 of the two logit rows, the unnormalised
// exponential sums l1, l2 and an accumulator acc of the P1-weighted logit
// difference -- finalised as KL = acc / l1 + LSE2 - LSE1, LSE_t = m_t + log l_t.
// The page does not print the per-tile update; the one used here (the only
// one for which that finaliser equals KL) is, for a tile of keys J:
//   m_t' = max(m_t, max_J s_t)            alpha_t = exp(m_t - m_t')
//   l_t  = alpha_t l_t + sum_J exp(s_t - m_t')
//   acc  = alpha_1 acc + sum_J exp(s_1 - m_1') (s_1 - s_2)
// Key tiles past a query block's causal frontier are never visited.
//
// Mapping to the hardware:
//   * one workgroup = 4 waves x 32 query rows; each wave keeps its queries'
//     Q1/Q2 fragments in registers for the whole key loop;
//   * K1/K2 tiles (64 keys for bf16, 32 for fp32) are staged in LDS, double
//     buffered through registers, with an XOR chunk swizzle;
//   * scores are computed transposed (S^T = K Q^T, 32x32 MFMA blocks) so each
//     lane owns ONE query and 16 keys of every 32-key block: the maxima and
//     sums are in-lane, each lane-half keeps its own five scalars and the two
//     halves are merged once, after the loop (the merge is the same rescale);
//   * exponentials are exp2 with scale*log2(e) folded into one FMA; the
//     maxima are tracked on raw dot products and scale is applied at the end.
#include "streamkl_device.h"
#include "streamkl_launch.h"

#include <climits>
#include <cmath>

namespace streamkl {
namespace {

template <bool BF16, int D>
struct FwdCfg {
  using G = RowGeom<BF16, D>;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBQ = 32 * kWaves;                 // queries per workgroup
  static constexpr int kBK = BF16 ? 64 : 32;              // keys per LDS tile
  static constexpr int kSub = kBK / 32;                   // 32-key blocks per tile
  static constexpr int kTileChunks = kBK * G::kChunks;    // 16-B chunks per tensor tile
  static constexpr int kLoads = kTileChunks / kThreads;   // chunks per thread per tensor
  static constexpr size_t kLdsBytes = size_t(2) * 2 * kTileChunks * 16;  // 2 stages x K1,K2
  static_assert(kTileChunks % kThreads == 0, "tile must split evenly over the workgroup");
};

struct FwdParams {
  const char *q1, *k1, *q2, *k2;
  float *kl, *lse1, *lse2;
  int nq, nk, nqb;
  float scale, c;  // c = scale * log2(e)
};

template <bool BF16, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  using C = FwdCfg<BF16, D>;
  using G = typename C::G;
  extern __shared__ u32x4 lds[];  // [stage][tensor][kTileChunks]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;

  // Heads are contiguous in logical order (one head per XCD at a time);
  // for causal problems the longest query blocks of a head go first.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = bid / p.nqb;
  const int qbr = bid - bh * p.nqb;
  const int qb = CAUSAL ? p.nqb - 1 - qbr : qbr;
  const int q0 = qb * C::kBQ;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + col;
  const bool wave_active = wq0 < p.nq;

  const size_t qoff = size_t(bh) * p.nq * G::kRowBytes;
  const size_t koff = size_t(bh) * p.nk * G::kRowBytes;

  // Stationary query fragments (B operand), zero for rows past N_Q.
  u32x4 qf1[G::kLaneChunks], qf2[G::kLaneChunks];
  if (qrow < p.nq) {
    const u32x4 *r1 = reinterpret_cast<const u32x4 *>(p.q1 + qoff + size_t(qrow) * G::kRowBytes);
    const u32x4 *r2 = reinterpret_cast<const u32x4 *>(p.q2 + qoff + size_t(qrow) * G::kRowBytes);
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) {
      qf1[c] = r1[frag_chunk<BF16, D>(h, c)];
      qf2[c] = r2[frag_chunk<BF16, D>(h, c)];
    }
  } else {
#pragma unroll
    for (int c = 0; c < G::kLaneChunks; ++c) qf1[c] = qf2[c] = zero4();
  }

  // Key range: [0, kend).  Causal: the last allowed key of row i is i + N_K - N_Q.
  const int off = p.nk - p.nq;
  int kend = p.nk;
  if (CAUSAL) kend = min(p.nk, min(q0 + C::kBQ, p.nq) + off);
  const int ntiles = (kend + C::kBK - 1) / C::kBK;
  const int my_last = CAUSAL ? min(qrow + off, p.nk - 1) : p.nk - 1;
  const int w_lo = CAUSAL ? min(wq0 + off, p.nk - 1) : p.nk - 1;       // smallest in the wave
  const int w_hi = CAUSAL ? min(wq0 + 31 + off, p.nk - 1) : p.nk - 1;  // largest in the wave

  const char *kb1 = p.k1 + koff;
  const char *kb2 = p.k2 + koff;

  // Stage key tile kt into LDS buffer `stage` with direct global->LDS copies.
  // Lane L of wave w fills chunk position p = i*256 + 64w + L of the tile;
  // the global side picks the (row, logical chunk) that belongs there under
  // the XOR swizzle (which is its own inverse).  Rows past N_K repeat the
  // last key; the compute masks them.
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int pos = i * C::kThreads + tid;
      const int row = pos / G::kChunks;
      const int ch = swz<G::kChunks>(row, pos % G::kChunks);
      const int key = min(kt * C::kBK + row, p.nk - 1);
      const size_t o = size_t(key) * G::kRowBytes + ch * 16;
      u32x4 *w1 = lds + (stage * 2 + 0) * C::kTileChunks + i * C::kThreads + wave * 64;
      u32x4 *w2 = lds + (stage * 2 + 1) * C::kTileChunks + i * C::kThreads + wave * 64;
      dma16(kb1 + o, w1);
      dma16(kb2 + o, w2);
    }
  };

  const float c = p.c;
  float m1 = -INFINITY, m2 = -INFINITY, l1 = 0.f, l2 = 0.f, acc = 0.f;

  if (ntiles > 0) issue(0, 0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int stage = kt & 1;
    // Buffer stage^1 was last read in iteration kt-1, which ended in a barrier.
    if (kt + 1 < ntiles) issue(kt + 1, stage ^ 1);
    const int kbase = kt * C::kBK;

    if (wave_active && kbase <= w_hi) {
      const u32x4 *b1 = lds + (stage * 2 + 0) * C::kTileChunks;
      const u32x4 *b2 = lds + (stage * 2 + 1) * C::kTileChunks;
      f32x16 s1[C::kSub], s2[C::kSub];
#pragma unroll
      for (int sb = 0; sb < C::kSub; ++sb) {
        s1[sb] = f32x16{};
        s2[sb] = f32x16{};
        const int row = sb * 32 + col;
#pragma unroll
        for (int cc = 0; cc < G::kLaneChunks; ++cc) {
          const int pos = row * G::kChunks + swz<G::kChunks>(row, frag_chunk<BF16, D>(h, cc));
          mfma_chunk<BF16>(b1[pos], qf1[cc], s1[sb]);
          mfma_chunk<BF16>(b2[pos], qf2[cc], s2[sb]);
        }
      }

      // Does any element of this tile lie past some row's last key?
      const bool need_mask = kbase + C::kBK - 1 > w_lo;
      float tm1 = m1, tm2 = m2;
      if (!need_mask) {
#pragma unroll
        for (int sb = 0; sb < C::kSub; ++sb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            tm1 = vmax3(s1[sb][r], s1[sb][r + 1], tm1);
            tm2 = vmax3(s2[sb][r], s2[sb][r + 1], tm2);
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < C::kSub; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = kbase + sb * 32 + c_row(r, h) <= my_last;
            tm1 = vmax(tm1, ok ? s1[sb][r] : -INFINITY);
            tm2 = vmax(tm2, ok ? s2[sb][r] : -INFINITY);
          }
      }
      const float m1n = tm1, m2n = tm2;
      const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2((m1 - m1n) * c);
      const float a2 = (m2 == -INFINITY) ? 0.f : fast_exp2((m2 - m2n) * c);
      const float nm1c = -m1n * c, nm2c = -m2n * c;

      float ts1a = 0.f, ts1b = 0.f, ts2a = 0.f, ts2b = 0.f, ta = 0.f, tb = 0.f;
      if (!need_mask) {
#pragma unroll
        for (int sb = 0; sb < C::kSub; ++sb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p1a = fast_exp2(fmaf(s1[sb][r], c, nm1c));
            const float p2a = fast_exp2(fmaf(s2[sb][r], c, nm2c));
            const float p1b = fast_exp2(fmaf(s1[sb][r + 1], c, nm1c));
            const float p2b = fast_exp2(fmaf(s2[sb][r + 1], c, nm2c));
            ts1a += p1a;
            ts2a += p2a;
            ts1b += p1b;
            ts2b += p2b;
            ta = fmaf(p1a, s1[sb][r] - s2[sb][r], ta);
            tb = fmaf(p1b, s1[sb][r + 1] - s2[sb][r + 1], tb);
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < C::kSub; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = kbase + sb * 32 + c_row(r, h) <= my_last;
            const float e1 = fast_exp2(fmaf(s1[sb][r], c, nm1c));
            const float e2 = fast_exp2(fmaf(s2[sb][r], c, nm2c));
            const float p1 = ok ? e1 : 0.f;
            const float p2 = ok ? e2 : 0.f;
            ts1a += p1;
            ts2a += p2;
            ta = fmaf(p1, s1[sb][r] - s2[sb][r], ta);
          }
      }
      l1 = fmaf(l1, a1, ts1a + ts1b);
      l2 = fmaf(l2, a2, ts2a + ts2b);
      acc = fmaf(acc, a1, ta + tb);
      m1 = m1n;
      m2 = m2n;
    }

    __syncthreads();  // also waits for the copies into stage^1
  }

  // Merge the two lane-halves (disjoint key subsets of the same query).
  const float om1 = __shfl_xor(m1, 32), om2 = __shfl_xor(m2, 32);
  const float ol1 = __shfl_xor(l1, 32), ol2 = __shfl_xor(l2, 32);
  const float oacc = __shfl_xor(acc, 32);
  const float M1 = vmax(m1, om1), M2 = vmax(m2, om2);
  const float fa1 = (m1 == -INFINITY) ? 0.f : fast_exp2((m1 - M1) * c);
  const float fb1 = (om1 == -INFINITY) ? 0.f : fast_exp2((om1 - M1) * c);
  const float fa2 = (m2 == -INFINITY) ? 0.f : fast_exp2((m2 - M2) * c);
  const float fb2 = (om2 == -INFINITY) ? 0.f : fast_exp2((om2 - M2) * c);
  const float L1 = l1 * fa1 + ol1 * fb1;
  const float L2 = l2 * fa2 + ol2 * fb2;
  const float A = acc * fa1 + oacc * fb1;

  if (h == 0 && qrow < p.nq) {
    const float lse1 = M1 * p.scale + logf(L1);
    const float lse2 = M2 * p.scale + logf(L2);
    const size_t o = size_t(bh) * p.nq + qrow;
    p.kl[o] = p.scale * (A / L1) + lse2 - lse1;
    p.lse1[o] = lse1;
    p.lse2[o] = lse2;
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
  using C = FwdCfg<BF16, D>;
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
  const long long blocks = (long long)p.nqb * a.bh;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  void *args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void *>(&fwd_kernel<BF16, D, CAUSAL>),
                         dim3(unsigned(blocks)), dim3(C::kThreads), args, C::kLdsBytes, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
  if (a.bf16) {
    if (a.d == 64) return a.causal ? launch<true, 64, true>(a, stream) : launch<true, 64, false>(a, stream);
    return a.causal ? launch<true, 128, true>(a, stream) : launch<true, 128, false>(a, stream);
  }
  if (a.d == 64) return a.causal ? launch<false, 64, true>(a, stream) : launch<false, 64, false>(a, stream);
  return a.causal ? launch<false, 128, true>(a, stream) : launch<false, 128, false>(a, stream);
}

}  // namespace streamkl
