// Backward pass, bf16 (placeholder until the tiled kernels land).
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
hipError_t launch_bwd_bf16(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
