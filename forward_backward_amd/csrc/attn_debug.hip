// Self-test of the debug build's address checks (-DATTN_DEBUG): one wave whose
// lanes check the 16-byte accesses at base + 16 * lane against the ranges the
// host registered, reading nothing. In a release build the check is empty.
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

__global__ __launch_bounds__(64) void attn_debug_selftest_kernel(const char* base) {
  ATTN_DBG_CHECK(base + 16 * threadIdx.x, 16);
}

}  // namespace

hipError_t launch_debug_selftest(const void* base, hipStream_t s) {
  hipLaunchKernelGGL(attn_debug_selftest_kernel, dim3(1), dim3(64), 0, s, static_cast<const char*>(base));
  return hipGetLastError();
}

}  // namespace attn
