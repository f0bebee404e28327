// streamkl_bwd_dq.hip -- query-gradient kernel of the recompute backward:
// each workgroup owns 128 query rows and streams key tiles up to its causal
// frontier, accumulating dQ1, dQ2 in registers (see streamkl_bwd.h).
#include "streamkl_bwd.h"

namespace streamkl {
hipError_t launch_bwd_dq(const BwdArgs &a, hipStream_t stream) { return launch_bwd_role<ROLE_DQ>(a, stream); }
}  // namespace streamkl
