// Attention backward for gfx950 (placeholder until the recomputation kernels land).
#include "launch.h"

namespace fa {

hipError_t launch_bwd(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
