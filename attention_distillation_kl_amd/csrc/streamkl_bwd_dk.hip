// streamkl_bwd_dk.hip -- key-gradient kernel of the recompute backward: each
// workgroup owns a block of key rows (256 for bf16, 64 in the paired form
// that small grids take) and streams query tiles from its causal frontier to
// N_Q, accumulating dK1, dK2 in registers (see streamkl_bwd.h).
#include "streamkl_bwd.h"

namespace streamkl {
hipError_t launch_bwd_dk(const BwdArgs &a, hipStream_t stream) { return launch_bwd_role<ROLE_DK>(a, stream); }
}  // namespace streamkl
