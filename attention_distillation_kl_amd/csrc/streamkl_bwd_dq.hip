// streamkl_bwd_dq.hip -- query-gradient kernel of the recompute backward:
// each workgroup owns a block of query rows and streams key tiles up to its
// causal frontier, accumulating dQ1, dQ2 in registers (see streamkl_bwd.h).
// For short query blocks the key tiles are partitioned over several
// workgroups per query block, whose partial sums a second kernel adds.
#include "streamkl_bwd.h"

#include <algorithm>

namespace streamkl {

hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t stream) { return launch_bwd_role<ROLE_DQ>(a, stream); }

int bwd_dq_default_splits(int bh, int nq, int nk, int d, bool bf16, int grad_mask) {
  // A workgroup of this kernel occupies a whole CU (its LDS), so grids with
  // at least one workgroup per CU are not split (measured: two partitions of
  // 256 workgroups are slower than none).  Smaller grids get partitions for
  // one round of workgroups (one per CU), each partition keeping at least
  // four key tiles (measured 1-2% faster than two rounds, with half the
  // workspace).
  constexpr long long kCUs = 256;
  if (bh <= 0 || nq <= 0 || nk <= 0) return 1;
  int bs, bt;
  auto pick = [&](auto bf16_c, auto d_c) {
    constexpr bool B = decltype(bf16_c)::value;
    constexpr int DD = decltype(d_c)::value;
    using C3 = BwdCfgOf<B, DD, 3, ROLE_DQ>;
    using C1 = BwdCfgOf<B, DD, 1, ROLE_DQ>;
    bs = grad_mask == 3 ? C3::kBS : C1::kBS;
    bt = C3::kBT;
  };
  if (bf16) {
    if (d == 64) pick(std::true_type{}, std::integral_constant<int, 64>{});
    else pick(std::true_type{}, std::integral_constant<int, 128>{});
  } else {
    if (d == 64) pick(std::false_type{}, std::integral_constant<int, 64>{});
    else pick(std::false_type{}, std::integral_constant<int, 128>{});
  }
  const long long nwg = (long long)bh * ((nq + bs - 1) / bs);
  constexpr long long kTarget = kCUs;
  if (nwg >= kCUs) return 1;
  const long long tiles = (nk + bt - 1) / bt;
  long long s = (kTarget + nwg - 1) / nwg;
  s = std::min(s, std::max(1LL, tiles / 4));
  return int(std::min(s, 256LL));
}

size_t bwd_dq_workspace_floats(int bh, int nq, int d, int grad_mask, int splits) {
  if (splits <= 1 || bh <= 0 || nq <= 0) return 0;
  const int ngrad = ((grad_mask & 1) ? 1 : 0) + ((grad_mask & 2) ? 1 : 0);
  return size_t(splits) * size_t(bh) * size_t(nq) * size_t(d) * size_t(ngrad);
}

#ifdef STREAMKL_DEBUG
unsigned dbg_take_bwd_dq() { return dbg_take(); }
#endif
}  // namespace streamkl
