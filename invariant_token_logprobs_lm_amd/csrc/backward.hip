// Gradient of the REINFORCE Zero loss through the LM head (not yet built:
// the entry point reports ITL_ERR_UNSUPPORTED).
#include "itl_launch.h"

namespace itl {

size_t backward_workspace_bytes(long long, long long, long long) { return 0; }

hipError_t launch_reinforce_zero_backward(const void*, const void*, int, int, int, int, const int32_t*, const float*,
                                          const float*, float*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace itl
