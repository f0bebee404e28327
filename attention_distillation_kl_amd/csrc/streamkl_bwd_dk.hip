// streamkl_bwd_dk.hip -- key-gradient kernel of the recompute backward: each
// workgroup owns a block of key rows (256 for bf16, 64 in the paired form
// that small grids take) and streams query tiles from its causal frontier to
// N_Q, accumulating dK1, dK2 in registers (see streamkl_bwd.h).
#include "streamkl_bwd.h"

#include <algorithm>

namespace streamkl {
hipError_t launch_bwd_dk(const BwdArgs &a, hipStream_t stream) { return launch_bwd_role<ROLE_DK>(a, stream); }

int bwd_dk_default_splits(int bh, int nq, int nk, int d, bool bf16, int grad_mask) {
  // A grid with fewer key blocks than resident workgroups, whose blocks
  // stream many query tiles, is bound by its longest blocks.  The query
  // range of every key block is then cut into equal runs, as many as fill
  // one round of resident workgroups, each at least 16 tiles long.  Measured
  // (one box, key half with its reduction): 1 head x 8K causal d = 128
  // 0.181 -> 0.084 ms, 2 heads x 4K queries x 2K keys 0.102 -> 0.052 ms,
  // 8 heads x 8K queries x 1K keys d = 64 0.146 -> 0.077 ms, C2's 8 heads x
  // 2K causal d = 64 -5%.  Two rounds were no better; runs of 8 tiles made
  // 16 heads x 1K causal d = 64 14% slower.  Grids that fill a round already
  // are not split.
  if (bh <= 0 || nq <= 0 || nk <= 0) return 1;
  const bool po = bwd_dk_paired(bh, nq, nk, bf16) && bf16;
  int bs = 0, bt = 0, per_cu = 0;
  auto pick = [&](auto bf16_c, auto d_c) {
    constexpr bool B = decltype(bf16_c)::value;
    constexpr int DD = decltype(d_c)::value;
    // Both gradients take the paired layout where it is chosen, one gradient
    // the unpaired one (with the paired block order for the student's).
    auto set = [&](auto cfg) {
      using C = decltype(cfg);
      bs = C::kBS;
      bt = C::kBT;
      per_cu = 4 * C::kWavesPerEU / C::kWaves;
    };
    if (grad_mask == 3 && po) set(BwdCfgOf<B, DD, 3, ROLE_DK, true>{});
    else if (grad_mask == 3) set(BwdCfgOf<B, DD, 3, ROLE_DK, false>{});
    else set(BwdCfgOf<B, DD, 1, ROLE_DK, false>{});
  };
  if (bf16) {
    if (d == 64) pick(std::true_type{}, std::integral_constant<int, 64>{});
    else pick(std::true_type{}, std::integral_constant<int, 128>{});
  } else {
    if (d == 64) pick(std::false_type{}, std::integral_constant<int, 64>{});
    else pick(std::false_type{}, std::integral_constant<int, 128>{});
  }
  constexpr long long kCUs = 256;
  const long long slots = kCUs * per_cu;
  const long long nwg = (long long)bh * ((nk + bs - 1) / bs);
  if (nwg >= slots) return 1;
  const long long tiles = (nq + bt - 1) / bt;
  long long s = (slots + nwg - 1) / nwg;
  s = std::min(s, std::max(1LL, tiles / 16));
  return int(std::min(s, 64LL));
}

size_t bwd_dk_workspace_floats(int bh, int nk, int d, int grad_mask, int splits) {
  if (splits <= 1 || bh <= 0 || nk <= 0) return 0;
  const int ngrad = ((grad_mask & 1) ? 1 : 0) + ((grad_mask & 2) ? 1 : 0);
  return size_t(splits) * size_t(bh) * size_t(nk) * size_t(d) * size_t(ngrad);
}
#ifdef STREAMKL_DEBUG
unsigned dbg_take_bwd_dk() { return dbg_take(); }
#endif
}  // namespace streamkl
