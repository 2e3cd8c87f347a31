// Backward pass of exact attention for gfx950 (recompute-based).
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

hipError_t launch_bwd(const BwdArgs&) { return hipErrorNotSupported; }

}  // namespace attn
