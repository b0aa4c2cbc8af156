// Split-KV decode, bf16 (placeholder until the kernels land).
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
hipError_t launch_decode_bf16(const DecodeArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
