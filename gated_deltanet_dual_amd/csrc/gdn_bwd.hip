// gdn_bwd.hip -- reverse mode of the dual-stream forward (placeholder launcher).
#include "kernels.h"

namespace flare {

hipError_t launch_gdn_bwd(const BwdArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace flare
